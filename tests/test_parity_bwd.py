"""GPU parity of the backward (dQ, dK, dV) with the oracle.

Small problems: every element.  The 16-trajectory workload: O, LSE, dQ, dK
and dV of the longest trajectory (9,472 tokens) element by element, one test
per KV head with its four query heads (marked slow: 4.4 TFLOP of dense fp64
oracle work in all); dQ, dK and dV of the two shortest trajectories whole;
dQ on sampled rows of every trajectory (each row's gradient is computed alone
by the oracle); and for every segment the two invariants that hold at any
size: dK sums to zero over a segment and dV sums to the group's summed dO.
Tolerance: max|err| <= 1e-2 * max|ref| per gradient tensor (per compared
slice, which is never looser than per whole tensor).
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

from gpu_helpers import TOL_GRAD, device_inputs, max_abs, sample_rows

pytestmark = pytest.mark.gpu


def run_bwd(w):
    q, k, v, cu, sc, do = device_inputs(w)
    o, lse = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    dq, dk, dv = bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, w.block_size, w.scale,
                                   w.max_seqlen)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))


def rel_err(got, ref):
    return max_abs(got, ref) / max(float(np.max(np.abs(ref))), 1e-30)


SMALL = [
    ("staircase_two_traj", [96 + 5 * 32, 32 + 3 * 32], [5, 3], 32, 8, 128, 32),
    ("block_causal_ragged", [200, 77], [0, 0], 8, 2, 128, 32),
    ("causal_B1", [150], [0], 4, 4, 128, 1),
    ("full_B_eq_L", [90], [0], 4, 1, 128, 90),
    ("odd_B7_group3", [300], [0], 6, 2, 128, 7),
    ("staircase_B64_group8", [64 * 3 + 2 * 64], [2], 16, 2, 128, 64),
    ("staircase_B8_d64", [40 + 3 * 8, 8 * 9 + 7 * 8], [3, 7], 4, 2, 64, 8),
    ("staircase_no_prefix", [4 * 32], [4], 8, 8, 128, 32),
    ("with_empty_segment", [64, 0, 100], [0, 0, 0], 4, 2, 128, 16),
    ("mixed_S0_and_S", [96, 64 + 3 * 32, 128, 32 + 2 * 32, 45], [0, 3, 0, 2, 0], 8, 2, 128, 32),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    name, seqlens, copies, hq, hkv, d, B = case
    w = W.packed(name, "staircase_bwd", 200 + len(name), seqlens, copies, hq, hkv, d, B, "bf16",
                 with_do=True)
    dq, dk, dv = run_bwd(w)
    _, _, dQ, dK, dV = oracle.attention_bwd(w.q, w.k, w.v, w.do, w.cu_seqlens, w.s_copies,
                                            w.block_size, w.scale)
    errs = [rel_err(dq, dQ), rel_err(dk, dK), rel_err(dv, dV)]
    print(f"{name}: rel err dQ {errs[0]:.3g} dK {errs[1]:.3g} dV {errs[2]:.3g}")
    assert max(errs) <= TOL_GRAD, errs


@pytest.fixture(scope="module")
def big():
    w = W.staircase_bwd_16traj()
    return w, run_bwd(w)


def test_16traj_dq_sampled_rows(big):
    w, (dq, dk, dv) = big
    rows = sample_rows(w, np.random.default_rng(44), per_segment=3)
    dQ = oracle.attention_dq_rows(w.q, w.k, w.v, w.do, w.cu_seqlens, w.s_copies, w.block_size,
                                  w.scale, rows)
    err = max_abs(dq[rows], dQ[rows]) / float(np.max(np.abs(dQ[rows])))
    print(f"dQ on {len(rows)} rows: rel err {err:.3g}")
    assert err <= TOL_GRAD


def test_16traj_whole_segments(big):
    w, (dq, dk, dv) = big
    lens = np.diff(w.cu_seqlens)
    for s in np.argsort(lens)[:2]:
        a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        _, _, dQ, dK, dV = oracle.attention_bwd(w.q[a:b], w.k[a:b], w.v[a:b], w.do[a:b],
                                                [0, b - a], [int(w.s_copies[s])], w.block_size,
                                                w.scale)
        errs = [rel_err(dq[a:b], dQ), rel_err(dk[a:b], dK), rel_err(dv[a:b], dV)]
        print(f"segment {s} (L={b - a}): rel err dQ {errs[0]:.3g} dK {errs[1]:.3g} dV {errs[2]:.3g}")
        assert max(errs) <= TOL_GRAD, errs


@pytest.mark.slow
@pytest.mark.parametrize("g", range(8))
def test_16traj_longest_trajectory_whole(big, g):
    """Forward and backward of the longest trajectory for KV head g and its
    query heads, against the oracle run on exactly that slice (the other
    heads of the segment do not touch these outputs)."""
    w, (dq, dk, dv) = big
    s = int(np.argmax(np.diff(w.cu_seqlens)))
    a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
    grp = w.hq // w.hkv
    hs = slice(g * grp, (g + 1) * grp)
    O, LSE, dQ, dK, dV = oracle.attention_bwd(w.q[a:b, hs], w.k[a:b, g:g + 1], w.v[a:b, g:g + 1],
                                              w.do[a:b, hs], [0, b - a], [int(w.s_copies[s])],
                                              w.block_size, w.scale)
    o, lse = big_forward(w)
    eo, el = max_abs(o[a:b, hs], O), max_abs(lse[hs, a:b], LSE)
    errs = [rel_err(dq[a:b, hs], dQ), rel_err(dk[a:b, g:g + 1], dK), rel_err(dv[a:b, g:g + 1], dV)]
    print(f"segment {s} (L={b - a}) KV head {g}: max|dO| {eo:.3g} max|dLSE| {el:.3g}; rel err "
          f"dQ {errs[0]:.3g} dK {errs[1]:.3g} dV {errs[2]:.3g}")
    assert eo <= 1e-2 and el <= 1e-2, (eo, el)
    assert max(errs) <= TOL_GRAD, errs


_FWD = {}


def big_forward(w):
    """O and LSE of the 16-trajectory forward as float64 (computed once)."""
    if "o" not in _FWD:
        q, k, v, cu, sc, _ = device_inputs(w)
        o, lse = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
        torch.cuda.synchronize()
        _FWD["o"] = o.float().cpu().numpy().astype(np.float64)
        _FWD["lse"] = lse.cpu().numpy().astype(np.float64)
    return _FWD["o"], _FWD["lse"]


def test_16traj_invariants_every_segment(big):
    w, (dq, dk, dv) = big
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


def test_backward_is_deterministic():
    w = W.staircase_fwd_8traj()
    w.do = torch.from_numpy(np.random.default_rng(8).standard_normal(
        (w.total, w.hq, w.d), dtype=np.float32)).to(torch.bfloat16)
    q, k, v, cu, sc, do = device_inputs(w)
    o, lse = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    g1 = bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, w.block_size, w.scale, w.max_seqlen)
    g2 = bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, w.block_size, w.scale, w.max_seqlen)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
