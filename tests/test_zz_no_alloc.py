"""bca_decode_noalloc through the C ABI: the decode step on the library's own
per-GPU scratch must give exactly the bytes bca_decode gives with a caller
workspace (same kernels, same split plan), call after call -- here a long
cache, then a shorter one that reuses the scratch the first call left -- and
match the fp64 oracle within the bf16 tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

pytestmark = pytest.mark.gpu


def noalloc_call(q, k, v, scale, o, lse, num_splits=0):
    q_len, hq, d = q.shape
    kv_len, hkv = k.shape[0], k.shape[1]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = ctypes.c_void_p
    return bca.lib().bca_decode_noalloc(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
                                        P(o.data_ptr()), P(lse.data_ptr()), q_len, kv_len, hq,
                                        hkv, d, scale, bca.BCA_BF16, num_splits, stream)


def test_noalloc_decode_matches_workspace_decode_twice():
    dev = torch.device("cuda", 0)
    for prefix in (8192, 1024):  # the second call is smaller than the first
        w = W.decode_step(prefix)
        q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
        o_ref, lse_ref = bca.decode(q, k, v, w.scale)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((w.hq, q.shape[0]), float("nan"), device=dev)
        assert noalloc_call(q, k, v, w.scale, o, lse) == 0, bca.lib().bca_last_error()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), prefix
        O, LSE = oracle.decode(w.q, w.k, w.v, w.scale)
        eo = float(np.abs(o.float().cpu().numpy() - O).max())
        el = float(np.abs(lse.cpu().numpy() - LSE).max())
        print(f"P={prefix}: max|dO| {eo:.3g} max|dLSE| {el:.3g}")
        assert eo <= 1e-2 and el <= 1e-2


def test_noalloc_rejects_more_than_its_scratch():
    dev = torch.device("cuda", 0)
    w = W.decode_step(8192)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    o = torch.full_like(q, 3.0)
    lse = torch.full((w.hq, q.shape[0]), 3.0, device=dev)
    # 256 splits of 32 heads x 32 rows x 128 bf16 values: 64 MiB of partials
    assert noalloc_call(q, k, v, w.scale, o, lse, num_splits=256) == 5
    assert b"scratch" in bca.lib().bca_last_error()
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 3.0).all())
