"""Compute-balanced packing: the oracle's rule pinned to textbook facts, the
library's host routine against the oracle (exact, integers), and the packed
output consumed by the staircase forward on the GPU.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

from gpu_helpers import device_inputs


def lib_or_skip():
    import os
    if not os.path.exists(bca.LIB_PATH):
        pytest.skip("libbca.so not built")
    return bca.lib()


# --- the oracle's rule, pinned ---------------------------------------------

def test_lpt_textbook_instance():
    # Graham's instance: jobs 3,3,2,2,2 on two machines.  The greedy rule puts
    # 3 | 3, then 2 on the first (tie -> lower machine), 2 on the second, 2 on
    # the first: loads 7 and 5, while 6 | 6 ({3,3}, {2,2,2}) is optimal.
    bin_of, bin_cost, order, start = oracle.lpt([3, 3, 2, 2, 2], 2)
    assert bin_of.tolist() == [0, 1, 0, 1, 0]
    assert bin_cost.tolist() == [7, 5]
    assert order.tolist() == [0, 2, 4, 1, 3] and start.tolist() == [0, 3, 5]
    assert oracle.optimal_makespan([3, 3, 2, 2, 2], 2) == 6


@pytest.mark.parametrize("seed", range(12))
def test_lpt_within_graham_bound(seed):
    rng = np.random.default_rng(seed)
    n, m = int(rng.integers(1, 8)), int(rng.integers(1, 4))
    costs = rng.integers(1, 50, size=n).tolist()
    _, bin_cost, order, start = oracle.lpt(costs, m)
    opt = oracle.optimal_makespan(costs, m)
    assert sum(bin_cost) == sum(costs)
    assert sorted(order.tolist()) == list(range(n)) and start[-1] == n
    assert max(bin_cost) * 3 * m <= (4 * m - 1) * opt     # <= (4/3 - 1/(3m)) OPT
    assert max(bin_cost) >= opt


def test_optimal_makespan_brute_force_small():
    # an exact split exists: 5+4 = 6+3 = 9
    assert oracle.optimal_makespan([6, 5, 4, 3], 2) == 9
    assert oracle.optimal_makespan([7], 3) == 7
    assert oracle.optimal_makespan([], 2) == 0


# --- the library against the oracle -----------------------------------------

@pytest.mark.parametrize("L,S,B", [(10, 3, 2), (7, 0, 3), (96, 2, 16), (64, 0, 64), (40, 5, 8),
                                   (33, 0, 32), (0, 0, 4), (48, 6, 8)])
def test_trajectory_cost_counts_the_mask(L, S, B):
    lib_or_skip()
    want = oracle.trajectory_cost(L, S, B)
    assert bca.trajectory_cost(L, S, B) == want
    assert W.useful_pairs([L], [S], B) == want


def test_trajectory_cost_rejects_bad_shapes():
    lib_or_skip()
    assert bca.trajectory_cost(10, 3, 4) == -1      # P = -2
    assert bca.trajectory_cost(13, 2, 4) == -1      # P = 5 is not whole blocks
    assert bca.trajectory_cost(5, 0, 0) == -1


@pytest.mark.parametrize("seed,n,m", [(0, 16, 8), (1, 8, 3), (2, 30, 4), (3, 3, 5), (4, 1, 1),
                                      (5, 50, 7), (6, 0, 2)])
def test_pack_matches_oracle(seed, n, m):
    lib_or_skip()
    rng = np.random.default_rng(seed)
    B = 8
    prefix = B * rng.integers(0, 12, size=n)
    copies = rng.integers(0, 5, size=n)
    # a few exact cost ties
    if n >= 4:
        prefix[1], copies[1] = prefix[0], copies[0]
        prefix[3], copies[3] = prefix[2], copies[2]
    seqlens = prefix + copies * B
    got = bca.pack_balanced(seqlens, copies, B, m)
    costs = [oracle.trajectory_cost(int(L), int(S), B) for L, S in zip(seqlens, copies)]
    want = oracle.lpt(costs, m)
    for g, w_ in zip(got, want):
        assert np.array_equal(g, w_), (g, w_)


def test_pack_rejects_bad_input():
    lib_or_skip()
    with pytest.raises(bca.BcaError):
        bca.pack_balanced([10], [3], 4, 2)       # P < 0
    with pytest.raises(bca.BcaError):
        bca.pack_balanced([8], [0], 4, 0)        # no bins


# --- copy-group trajectories ------------------------------------------------

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden",
                                    "staircase_groups_allowed_L12_P6_B2.txt")


def test_group_cost_counts_the_hand_written_table():
    # The hand-written admitted-key table of a 12-token segment (groups
    # (pe 2, 1 copy) and (pe 4, 2 copies), B = 2) lists 56 admitted pairs.
    n = 0
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            n += len(line.split(":", 1)[1].split())
    assert n == 56
    assert oracle.trajectory_cost_groups(12, [(2, 1), (4, 2)], 2) == n
    lib_or_skip()
    assert bca.trajectory_cost_groups(12, [(2, 1), (4, 2)], 2) == n


def random_groups(rng, n, B):
    seqlens, groups = [], []
    for _ in range(n):
        nb = int(rng.integers(0, 7))
        gs, pe = [], 0
        for _ in range(int(rng.integers(0, 4))):
            pe = int(rng.integers(pe // B, nb + 1)) * B   # non-decreasing, in [0, P]
            gs.append((pe, int(rng.integers(0, 4))))
        groups.append(gs)
        seqlens.append(nb * B + B * sum(c for _, c in gs))
    return seqlens, groups


@pytest.mark.parametrize("seed", range(6))
def test_group_cost_and_packing_match_the_oracle(seed):
    lib_or_skip()
    rng = np.random.default_rng(100 + seed)
    B = 4
    seqlens, groups = random_groups(rng, int(rng.integers(1, 12)), B)
    costs = [oracle.trajectory_cost_groups(L, g, B) for L, g in zip(seqlens, groups)]
    assert [bca.trajectory_cost_groups(L, g, B) for L, g in zip(seqlens, groups)] == costs
    # one group seeing the whole prefix is the plain staircase
    assert W.useful_pairs_groups(seqlens, groups, B) == sum(costs)
    for m in (1, 2, 5):
        got = bca.pack_balanced_groups(seqlens, groups, B, m)
        want = oracle.lpt(costs, m)
        for g, w_ in zip(got, want):
            assert np.array_equal(g, w_), (seed, m)


def test_one_group_is_the_plain_staircase_cost():
    lib_or_skip()
    for L, S, B in ((96, 2, 16), (40, 5, 8), (48, 6, 8)):
        P = L - S * B
        assert bca.trajectory_cost_groups(L, [(P, S)], B) == bca.trajectory_cost(L, S, B)


def test_group_cost_rejects_bad_groups():
    lib_or_skip()
    assert bca.trajectory_cost_groups(12, [(3, 1)], 2) == -1          # pe not a multiple of B
    assert bca.trajectory_cost_groups(12, [(4, 2), (2, 1)], 2) == -1  # pe decreasing
    assert bca.trajectory_cost_groups(12, [(12, 1)], 2) == -1         # pe beyond P = 10
    assert bca.trajectory_cost_groups(12, [(0, 7)], 2) == -1          # P < 0
    assert bca.trajectory_cost_groups(12, [(0, -1)], 2) == -1         # negative copies
    with pytest.raises(bca.BcaError):
        bca.pack_balanced_groups([12, 8], [[(3, 1)], []], 2, 2)


# --- a GPU consumer of the packed output ----------------------------------

@pytest.mark.gpu
def test_packed_bins_reproduce_the_full_batch():
    """Repacking the 8 trajectories into 3 balanced bins and running each bin
    alone gives every trajectory bit-identical O and LSE rows."""
    w = W.staircase_fwd_8traj()
    q, k, v, cu, sc, _ = device_inputs(w)
    o_all, lse_all = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    lens = np.diff(w.cu_seqlens)
    bin_of, bin_cost, order, start = bca.pack_balanced(lens, w.s_copies, w.block_size, 3)
    costs = [bca.trajectory_cost(int(L), int(S), w.block_size) for L, S in zip(lens, w.s_copies)]
    assert max(bin_cost) * 9 <= 11 * oracle.optimal_makespan(costs, 3)  # LPT bound, m = 3
    for b in range(3):
        members = order[start[b]:start[b + 1]].tolist()
        if not members:
            continue
        rows = [torch.arange(int(w.cu_seqlens[t]), int(w.cu_seqlens[t + 1]), device=q.device)
                for t in members]
        idx = torch.cat(rows)
        cu_b = torch.tensor(np.concatenate([[0], np.cumsum([len(r) for r in rows])]),
                            dtype=torch.int32, device=q.device)
        sc_b = torch.tensor([int(w.s_copies[t]) for t in members], dtype=torch.int32,
                            device=q.device)
        max_len = max(len(r) for r in rows)
        o_b, lse_b = bca.staircase_fwd(q[idx].contiguous(), k[idx].contiguous(),
                                       v[idx].contiguous(), cu_b, sc_b, w.block_size, w.scale,
                                       max_len)
        torch.cuda.synchronize()
        assert torch.equal(o_b, o_all[idx])
        assert torch.equal(lse_b, lse_all[:, idx])


@pytest.mark.gpu
def test_packed_group_bins_reproduce_the_full_batch():
    """The copy-group workload repacked into 3 bins by compute: each bin run
    alone gives every trajectory bit-identical O, LSE, dQ, dK and dV rows."""
    w = W.staircase_groups_8traj()
    q, k, v, cu, _, do = device_inputs(w)
    dev = q.device
    gs, gp, gc = (torch.from_numpy(x).to(dev) for x in w.group_table())
    B = w.block_size
    o_all, lse_all = bca.staircase_groups_fwd(q, k, v, cu, gs, gp, gc, B, w.scale, w.max_seqlen)
    g_all = bca.staircase_groups_bwd(q, k, v, o_all, lse_all, do, cu, gs, gp, gc, B, w.scale,
                                     w.max_seqlen)
    lens = np.diff(w.cu_seqlens)
    bin_of, bin_cost, order, start = bca.pack_balanced_groups(lens, w.groups, B, 3)
    costs = [oracle.trajectory_cost_groups(int(L), g, B) for L, g in zip(lens, w.groups)]
    assert bin_cost.tolist() == oracle.lpt(costs, 3)[1].tolist()
    for b in range(3):
        members = order[start[b]:start[b + 1]].tolist()
        if not members:
            continue
        rows = [torch.arange(int(w.cu_seqlens[t]), int(w.cu_seqlens[t + 1]), device=dev)
                for t in members]
        idx = torch.cat(rows)
        cu_b = torch.tensor(np.concatenate([[0], np.cumsum([len(r) for r in rows])]),
                            dtype=torch.int32, device=dev)
        gs_b, gp_b, gc_b = (torch.from_numpy(x).to(dev)
                            for x in bca._group_arrays([w.groups[t] for t in members]))
        ml = max(len(r) for r in rows)
        qb, kb, vb, dob = (t[idx].contiguous() for t in (q, k, v, do))
        o_b, lse_b = bca.staircase_groups_fwd(qb, kb, vb, cu_b, gs_b, gp_b, gc_b, B, w.scale, ml)
        g_b = bca.staircase_groups_bwd(qb, kb, vb, o_b, lse_b, dob, cu_b, gs_b, gp_b, gc_b, B,
                                       w.scale, ml)
        torch.cuda.synchronize()
        assert torch.equal(o_b, o_all[idx]) and torch.equal(lse_b, lse_all[:, idx])
        for x_b, x_all in zip(g_b, g_all):
            assert torch.equal(x_b, x_all[idx]), b
