"""GPU parity of the general trajectory staircase (copy groups per block)
with the oracle: forward (bf16 and float32) and backward.

Small problems: every element.  The 8-trajectory workload: O, LSE, dQ, dK and
dV of every trajectory element by element (one test per trajectory, about 2.3
TFLOP of dense fp64 oracle work in all), plus per trajectory the invariants
that hold at any size (dK sums to zero over a segment, dV sums to the group's
summed dO).
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

from gpu_helpers import (TOL_BF16, TOL_F32, TOL_GRAD, device_inputs, group_tensors, max_abs,
                         run_groups_fwd)

pytestmark = pytest.mark.gpu


def make(name, seed, groups_per_seg, clean_blocks, hq, hkv, d, B, dtype="bf16", with_do=True):
    seqlens = [nb * B + B * sum(c for _, c in g) for nb, g in zip(clean_blocks, groups_per_seg)]
    copies = [sum(c for _, c in g) for g in groups_per_seg]
    w = W.packed(name, "staircase_groups", seed, seqlens, copies, hq, hkv, d, B, dtype,
                 with_do=with_do)
    w.groups = [list(g) for g in groups_per_seg]
    return w


SMALL = [
    # name, groups per segment, clean blocks per segment, hq, hkv, d, B
    ("every_block_B32", [[(0, 2), (32, 1), (64, 3), (96, 1)]], [4], 8, 2, 128, 32),
    ("two_traj_gqa4", [[(0, 1), (32, 2), (64, 1)], [(0, 3), (32, 1)]], [3, 2], 8, 2, 128, 32),
    ("repeated_pe", [[(64, 2), (64, 1), (128, 2)]], [4], 4, 4, 128, 32),
    ("B16_d64", [[(0, 1), (16, 2), (48, 3), (80, 1)]], [6], 4, 1, 64, 16),
    ("B64_group8", [[(0, 1), (64, 2), (128, 1)]], [3], 16, 2, 128, 64),
    ("no_groups_segment", [[(0, 2), (32, 1)], [], [(32, 2)]], [2, 3, 2], 4, 2, 128, 32),
    ("pe_zero_only", [[(0, 5)]], [3], 4, 2, 128, 32),
    ("B8_odd_tiles", [[(0, 3), (8, 2), (24, 4), (40, 1)]], [7], 8, 8, 128, 8),
    # long group tables: 64 and 65 groups in one segment (one per block)
    ("groups_64_one_segment", [[(4 * b, 1 + b % 2) for b in range(64)]], [64], 4, 2, 64, 4),
    ("groups_65_one_segment", [[(4 * b, 1 + (b % 3 == 0)) for b in range(65)]], [65], 4, 2, 64, 4),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_forward_and_backward(case):
    name, groups, clean, hq, hkv, d, B = case
    w = make(name, 300 + len(name), groups, clean, hq, hkv, d, B)
    o, lse = run_groups_fwd(w)
    O, LSE = oracle.attention_fwd(w.q, w.k, w.v, w.cu_seqlens, w.groups, B, w.scale)
    assert max_abs(o, O) <= TOL_BF16 and max_abs(lse, LSE) <= TOL_BF16
    q, k, v, cu, _, do = device_inputs(w)
    gs, gp, gc = group_tensors(w)
    o_d, lse_d = bca.staircase_groups_fwd(q, k, v, cu, gs, gp, gc, B, w.scale, w.max_seqlen)
    dq, dk, dv = bca.staircase_groups_bwd(q, k, v, o_d, lse_d, do, cu, gs, gp, gc, B, w.scale,
                                          w.max_seqlen)
    torch.cuda.synchronize()
    _, _, dQ, dK, dV = oracle.attention_bwd(w.q, w.k, w.v, w.do, w.cu_seqlens, w.groups, B,
                                            w.scale)
    for got, ref in ((dq, dQ), (dk, dK), (dv, dV)):
        got = got.float().cpu().numpy().astype(np.float64)
        assert max_abs(got, ref) <= TOL_GRAD * np.abs(ref).max(), name


def test_small_float32_forward():
    w = make("f32", 41, [[(0, 1), (16, 2), (32, 1)]], [3], 2, 1, 64, 16, dtype="f32",
             with_do=False)
    o, lse = run_groups_fwd(w)
    O, LSE = oracle.attention_fwd(w.q, w.k, w.v, w.cu_seqlens, w.groups, 16, w.scale)
    assert max_abs(o, O) <= TOL_F32 and max_abs(lse, LSE) <= TOL_F32


def test_one_group_equals_staircase_entry_point():
    w = W.staircase_fwd_8traj()
    P = w.prefix_lens
    w.groups = [[(int(p), int(s))] for p, s in zip(P, w.s_copies)]
    q, k, v, cu, sc, _ = device_inputs(w)
    gs, gp, gc = group_tensors(w)
    o1, l1 = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    o2, l2 = bca.staircase_groups_fwd(q, k, v, cu, gs, gp, gc, w.block_size, w.scale,
                                      w.max_seqlen)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.fixture(scope="module")
def big():
    w = W.staircase_groups_8traj()
    q, k, v, cu, _, do = device_inputs(w)
    gs, gp, gc = group_tensors(w)
    o, lse = bca.staircase_groups_fwd(q, k, v, cu, gs, gp, gc, w.block_size, w.scale,
                                      w.max_seqlen)
    dq, dk, dv = bca.staircase_groups_bwd(q, k, v, o, lse, do, cu, gs, gp, gc, w.block_size,
                                          w.scale, w.max_seqlen)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return w, f(o), lse.cpu().numpy().astype(np.float64), f(dq), f(dk), f(dv)


@pytest.mark.parametrize("s", range(8))
def test_8traj_every_trajectory_whole(big, s):
    w, o, lse, dq, dk, dv = big
    a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
    O, LSE, dQ, dK, dV = oracle.attention_bwd(w.q[a:b], w.k[a:b], w.v[a:b], w.do[a:b],
                                              [0, b - a], [w.groups[s]], w.block_size, w.scale)
    eo, el = max_abs(o[a:b], O), max_abs(lse[:, a:b], LSE)
    errs = [max_abs(got, ref) / np.abs(ref).max()
            for got, ref in ((dq[a:b], dQ), (dk[a:b], dK), (dv[a:b], dV))]
    print(f"segment {s} (L={b - a}, {len(w.groups[s])} groups): max|dO| {eo:.3g} "
          f"max|dLSE| {el:.3g}; rel err dQ {errs[0]:.3g} dK {errs[1]:.3g} dV {errs[2]:.3g}")
    assert eo <= TOL_BF16 and el <= TOL_BF16, (eo, el)
    assert max(errs) <= TOL_GRAD, errs


def test_8traj_invariants_every_segment(big):
    w, _, _, dq, dk, dv = big
    group = w.hq // w.hkv
    do = w.do.float().numpy().astype(np.float64)
    for s in range(w.nseq):
        a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        for g in range(w.hkv):
            sk = np.abs(dk[a:b, g].sum(0)).max()
            assert sk <= 1e-2 * np.abs(dk[a:b, g]).sum(0).max(), (s, g, sk)
            want = do[a:b, g * group:(g + 1) * group].sum((0, 1))
            sv = np.abs(dv[a:b, g].sum(0) - want).max()
            assert sv <= 1e-2 * np.abs(dv[a:b, g]).sum(0).max(), (s, g, sv)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
