"""Decode step against an FP8 E4M3 KV cache: GPU parity with the oracle on
the decoded cache (K = k_scale * e4m3(k8), V = v_scale * e4m3(v8)).

The GPU widens every E4M3 byte exactly to bf16 and folds the scales into the
softmax scale and the output, so the bf16 tolerance applies unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

from gpu_helpers import TOL_BF16, max_abs

pytestmark = pytest.mark.gpu


def run(P, num_splits=0, **kw):
    w, k8, v8, ks, vs = W.decode_step_fp8(P, **kw)
    dev = torch.device("cuda", 0)
    o, lse = bca.decode_fp8(w.q.to(dev), k8.to(dev), v8.to(dev), ks, vs, w.scale,
                            num_splits=num_splits)
    torch.cuda.synchronize()
    return w, k8, v8, ks, vs, o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy()


@pytest.mark.parametrize("P", [1024, 8192])
def test_fp8_decode_matches_oracle(P):
    w, k8, v8, ks, vs, o, lse = run(P)
    # the oracle decodes the bytes itself
    K = oracle.e4m3_to_float(k8.numpy()) * ks
    V = oracle.e4m3_to_float(v8.numpy()) * vs
    O, LSE = oracle.decode(w.q, K, V, w.scale)
    assert max_abs(o, O) <= TOL_BF16 and max_abs(lse, LSE) <= TOL_BF16


@pytest.mark.parametrize("P,B,hq,hkv,d", [(0, 32, 32, 8, 128), (100 * 2, 16, 4, 4, 128),
                                          (960, 32, 16, 2, 64), (250, 48, 6, 2, 128),
                                          (300, 40, 16, 8, 128)])
def test_fp8_decode_edge_shapes(P, B, hq, hkv, d):
    w, k8, v8, ks, vs, o, lse = run(P, block_size=B, hq=hq, hkv=hkv, d=d, seed=9)
    K = oracle.e4m3_to_float(k8.numpy()) * ks
    V = oracle.e4m3_to_float(v8.numpy()) * vs
    O, LSE = oracle.decode(w.q, K, V, w.scale)
    assert max_abs(o, O) <= TOL_BF16 and max_abs(lse, LSE) <= TOL_BF16


# Rounds of up to five key tiles per workgroup: 5 + 1 and 5 + 2 (129 tiles in
# 21 splits), 5 + 5 and 5 + 5 + 1 (32 tiles in 3 splits), against the oracle.
@pytest.mark.parametrize("P,ns", [(8192, 21), (2048 - 32, 3)])
def test_fp8_multi_round_splits_match_oracle(P, ns):
    w, k8, v8, ks, vs, o, lse = run(P, num_splits=ns)
    K = oracle.e4m3_to_float(k8.numpy()) * ks
    V = oracle.e4m3_to_float(v8.numpy()) * vs
    O, LSE = oracle.decode(w.q, K, V, w.scale)
    assert max_abs(o, O) <= TOL_BF16 and max_abs(lse, LSE) <= TOL_BF16


def test_fp8_split_invariance_and_determinism():
    ref = run(4096, num_splits=1)
    for ns in (3, 16, 0):
        got = run(4096, num_splits=ns)
        assert max_abs(got[5], ref[5]) <= 2.0 ** -8
        assert max_abs(got[6], ref[6]) <= 1e-5
    again = run(4096)
    assert np.array_equal(again[5], run(4096)[5])


def test_fp8_rejects_bad_scales_and_dtypes():
    w, k8, v8, ks, vs = W.decode_step_fp8(64)
    dev = torch.device("cuda", 0)
    q, k8, v8 = w.q.to(dev), k8.to(dev), v8.to(dev)
    with pytest.raises(bca.BcaError):
        bca.decode_fp8(q, k8, v8, 0.0, vs)
    with pytest.raises(bca.BcaError):
        bca.decode_fp8(q.float(), k8, v8, ks, vs)
