"""GPU parity of the forward kernels (block-causal and staircase) with the oracle.

Every comparison is element by element on every row and head: the small
problems, the 4096-token prefill, the 8-trajectory staircase (one test per
trajectory) and the 16-trajectory staircase (one test per trajectory, marked
slow: about 12 TFLOP of dense fp64 oracle work in all).  A sampled-row check
of the 16-trajectory workload (segment and block edges, the prefix/copy
boundary and random rows) stays as the quick version of the last.
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

from gpu_helpers import (TOL_BF16, TOL_F32, device_inputs, max_abs, oracle_rows, run_fwd,
                         sample_rows)

pytestmark = pytest.mark.gpu


def full_check(w, tol):
    o, lse = run_fwd(w)
    O, LSE = oracle.attention_fwd(w.q, w.k, w.v, w.cu_seqlens, w.s_copies, w.block_size, w.scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    eo, el = max_abs(o, O), max_abs(lse, LSE)
    print(f"{w.name}: max|dO| = {eo:.3g}, max|dLSE| = {el:.3g}")
    assert eo <= tol, eo
    assert el <= tol, el


def test_fp32_block_causal_L256_d64():
    full_check(W.blockcausal_fp32_small(), TOL_F32)


SMALL = [
    # name, seqlens, copies, hq, hkv, d, B, dtype
    ("ragged_L200_gqa4", [200], [0], 4, 1, 128, 32, "bf16"),
    ("packed_with_empty_d64", [77, 0, 130, 64], [0, 0, 0, 0], 8, 2, 64, 16, "bf16"),
    ("causal_B1", [300], [0], 2, 2, 128, 1, "bf16"),
    ("full_B_eq_L_mha", [150], [0], 3, 3, 64, 150, "bf16"),
    ("B_gt_L", [90], [0], 4, 2, 128, 128, "bf16"),
    ("staircase_two_traj", [96 + 5 * 32, 32 + 3 * 32], [5, 3], 32, 8, 128, 32, "bf16"),
    ("staircase_no_prefix", [4 * 32], [4], 8, 8, 128, 32, "bf16"),
    ("staircase_B64_group8", [64 * 3 + 2 * 64], [2], 16, 2, 128, 64, "bf16"),
    ("staircase_B8_group2", [40 + 3 * 8, 8 * 9 + 7 * 8], [3, 7], 6, 3, 64, 8, "bf16"),
    ("odd_B7_group3", [1000], [0], 12, 4, 128, 7, "bf16"),
    ("single_token", [1, 1, 2], [0, 0, 0], 4, 4, 128, 32, "bf16"),
    ("f32_packed_gqa", [200, 57], [0, 0], 4, 2, 128, 16, "f32"),
    ("f32_staircase", [40 + 3 * 8], [3], 2, 1, 64, 8, "f32"),
    # segments without copies packed next to staircase segments
    ("mixed_S0_and_S", [96, 64 + 3 * 32, 128, 32 + 2 * 32, 45], [0, 3, 0, 2, 0], 8, 2, 128, 32,
     "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    name, seqlens, copies, hq, hkv, d, B, dt = case
    w = W.packed(name, "staircase_fwd", 100 + len(name), seqlens, copies, hq, hkv, d, B, dt)
    full_check(w, TOL_F32 if dt == "f32" else TOL_BF16)


def test_block_causal_entry_equals_staircase_without_copies():
    w = W.packed("bc", "fwd", 7, [333, 64], [0, 0], 8, 2, 128, 32, "bf16")
    o1, l1 = run_fwd(w, staircase=True)
    o2, l2 = run_fwd(w, staircase=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def sampled_check(w, seed):
    rng = np.random.default_rng(seed)
    o, lse = run_fwd(w)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = sample_rows(w, rng)
    O, LSE = oracle_rows(w, rows)
    eo = max_abs(o[rows], O[rows])
    el = max_abs(lse[:, rows], LSE[:, rows])
    print(f"{w.name}: {len(rows)} rows x {w.hq} heads, max|dO| = {eo:.3g}, max|dLSE| = {el:.3g}")
    assert eo <= TOL_BF16, eo
    assert el <= TOL_BF16, el


def test_prefill_4k_every_row():
    full_check(W.prefill_bf16_4k(), TOL_BF16)


_GPU_FWD = {}


def gpu_forward(name, make):
    """The GPU forward of a named workload, computed once per test module."""
    if name not in _GPU_FWD:
        w = make()
        _GPU_FWD[name] = (w,) + run_fwd(w)
    return _GPU_FWD[name]


def segment_check(w, o, lse, s):
    """Every row and head of segment s against the oracle run on that segment alone."""
    a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
    O, LSE = oracle.attention_fwd(w.q[a:b], w.k[a:b], w.v[a:b], [0, b - a], [int(w.s_copies[s])],
                                  w.block_size, w.scale)
    assert np.isfinite(o[a:b]).all() and np.isfinite(lse[:, a:b]).all()
    eo, el = max_abs(o[a:b], O), max_abs(lse[:, a:b], LSE)
    print(f"{w.name} segment {s} (L={b - a}, S={int(w.s_copies[s])}): max|dO| = {eo:.3g}, "
          f"max|dLSE| = {el:.3g}")
    assert eo <= TOL_BF16, eo
    assert el <= TOL_BF16, el


@pytest.mark.parametrize("s", range(8))
def test_staircase_8traj_every_row(s):
    w, o, lse = gpu_forward("8traj", W.staircase_fwd_8traj)
    segment_check(w, o, lse, s)


@pytest.mark.slow
@pytest.mark.parametrize("s", range(16))
def test_staircase_16traj_every_row(s):
    w, o, lse = gpu_forward("16traj", W.staircase_bwd_16traj)
    segment_check(w, o, lse, s)


def test_staircase_16traj_forward_sampled():
    sampled_check(W.staircase_bwd_16traj(), 4)


def test_forward_is_deterministic():
    w = W.prefill_bf16_4k()
    q, k, v, cu, sc, _ = device_inputs(w)
    o1, l1 = bca.fwd(q, k, v, cu, w.block_size, w.scale, w.max_seqlen)
    o2, l2 = bca.fwd(q, k, v, cu, w.block_size, w.scale, w.max_seqlen)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_every_row_written():
    # Outputs pre-filled with NaN must come back finite on every row.
    w = W.staircase_fwd_8traj()
    q, k, v, cu, sc, _ = device_inputs(w)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.hq, w.total), float("nan"), device=q.device)
    bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
