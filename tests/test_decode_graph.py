"""The captured decode loop (bca_decode_graph_*) against eager decode calls.

A graph of several decode steps is replayed three times; before each replay
new queries and new own-block K/V rows are written into the captured buffers
(eager work, with synchronisation in between), and every replay's O and LSE
must equal, bit for bit, an eager bca_decode on the same inputs (same kernels,
same split plan, deterministic), and match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

from gpu_helpers import TOL_BF16, max_abs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P,steps", [(1024, 4), (256, 1)])
def test_graph_replays_match_eager(P, steps):
    w = W.decode_step(P, seed=11)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    g = bca.DecodeGraph(q, k, v, steps, w.scale)
    rng = np.random.default_rng(12)
    B = w.block_size
    try:
        for rep in range(3):
            # a new denoising step: new queries and new own-block keys/values
            q.copy_(torch.from_numpy(rng.standard_normal(tuple(q.shape), dtype=np.float32)))
            k[-B:].copy_(torch.from_numpy(rng.standard_normal((B,) + tuple(k.shape[1:]),
                                                              dtype=np.float32)))
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            o_g, l_g = g.out.clone(), g.lse.clone()
            o_e, l_e = bca.decode(q, k, v, w.scale)
            torch.cuda.synchronize()
            assert torch.equal(o_g, o_e), rep
            assert torch.equal(l_g, l_e), rep
            O, LSE = oracle.decode(q.cpu(), k.cpu(), v.cpu(), w.scale)
            o = o_g.float().cpu().numpy().astype(np.float64)
            lse = l_g.cpu().numpy().astype(np.float64)
            assert max_abs(o, O) <= TOL_BF16 and max_abs(lse, LSE) <= TOL_BF16
    finally:
        g.close()


def test_graph_launch_after_close_is_rejected():
    w = W.decode_step(64, seed=13)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    g = bca.DecodeGraph(q, k, v, 2, w.scale)
    g.launch()
    g.close()
    with pytest.raises(bca.BcaError):
        g.launch()


def _oracle_check(q, k, v, scale, o, lse):
    O, LSE = oracle.decode(q.cpu(), k.cpu(), v.cpu(), scale)
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert max_abs(o, O) <= TOL_BF16 and max_abs(lse, LSE) <= TOL_BF16


# (requested splits, device-resident lengths written before successive replays):
# full capacity, a shorter prefix, fewer tiles than splits (empty splits),
# one ragged tile, and values clamped to [q_len, capacity].
@pytest.mark.parametrize("num_splits", [16, 0])
def test_loop_follows_the_device_resident_length(num_splits):
    B, steps, cap = 32, 4, 2080
    w = W.decode_step(cap - B, seed=21)
    dev = torch.device("cuda", 0)
    k, v = w.k.to(dev), w.v.to(dev)
    rng = np.random.default_rng(22)
    q = torch.from_numpy(rng.standard_normal((steps,) + tuple(w.q.shape), dtype=np.float32))
    q = q.to(torch.bfloat16).to(dev)
    kv_len = torch.full((1,), cap, dtype=torch.int32, device=dev)
    loop = bca.DecodeLoop(q, k, v, kv_len, w.scale, num_splits=num_splits)
    try:
        for L in (2080, 1056, 544, 40, 5000, 10):
            Lc = min(max(L, B), cap)
            kv_len.fill_(L)
            q.copy_(torch.from_numpy(rng.standard_normal(tuple(q.shape), dtype=np.float32)))
            # the block's own rows are the last q_len rows of the attended cache
            k[Lc - B:Lc].copy_(torch.from_numpy(
                rng.standard_normal((B,) + tuple(k.shape[1:]), dtype=np.float32)))
            torch.cuda.synchronize()
            loop.launch()
            torch.cuda.synchronize()
            o_g, l_g = loop.out.clone(), loop.lse.clone()
            for i in range(steps):
                if num_splits and (Lc + 63) // 64 > 1:
                    # same tiles per split (eager caps the split count at the
                    # tile count; the loop's extra splits are empty, weight 0)
                    o_e, l_e = bca.decode(q[i], k[:Lc], v[:Lc], w.scale, num_splits=num_splits)
                    torch.cuda.synchronize()
                    assert torch.equal(o_g[i], o_e), (L, i)
                    assert torch.equal(l_g[i], l_e), (L, i)
                _oracle_check(q[i], k[:Lc], v[:Lc], w.scale, o_g[i], l_g[i])
    finally:
        loop.close()


def test_loop_runs_the_device_resident_step_count():
    """Only the first steps_dev[0] steps of a replay run; later steps leave
    their outputs as they were (here NaN), and the steps that run equal a
    replay of the whole loop."""
    B, steps, cap = 32, 4, 1056
    w = W.decode_step(cap - B, seed=23)
    dev = torch.device("cuda", 0)
    k, v = w.k.to(dev), w.v.to(dev)
    rng = np.random.default_rng(24)
    q = torch.from_numpy(rng.standard_normal((steps,) + tuple(w.q.shape), dtype=np.float32))
    q = q.to(torch.bfloat16).to(dev)
    kv_len = torch.full((1,), cap, dtype=torch.int32, device=dev)
    n_steps = torch.full((1,), steps, dtype=torch.int32, device=dev)
    loop = bca.DecodeLoop(q, k, v, kv_len, w.scale, steps_dev=n_steps)
    try:
        loop.launch()
        torch.cuda.synchronize()
        o_all, l_all = loop.out.clone(), loop.lse.clone()
        for n in (2, 0, 3):
            loop.out.fill_(float("nan"))
            loop.lse.fill_(float("nan"))
            n_steps.fill_(n)
            torch.cuda.synchronize()
            loop.launch()
            torch.cuda.synchronize()
            assert torch.equal(loop.out[:n], o_all[:n]) and torch.equal(loop.lse[:n], l_all[:n])
            assert torch.isnan(loop.out[n:].float()).all() and torch.isnan(loop.lse[n:]).all()
    finally:
        loop.close()


@pytest.mark.parametrize("cap,num_splits", [(96, 1), (64, 0)])
def test_loop_single_split_with_shorter_cache(cap, num_splits):
    """One split (no partials, the decode kernel writes O itself) with the
    device-resident length below the capacity: rows past it are masked."""
    B, steps = 32, 2
    w = W.decode_step(cap - B, seed=25)
    dev = torch.device("cuda", 0)
    k, v = w.k.to(dev), w.v.to(dev)
    rng = np.random.default_rng(26)
    q = torch.from_numpy(rng.standard_normal((steps,) + tuple(w.q.shape), dtype=np.float32))
    q = q.to(torch.bfloat16).to(dev)
    kv_len = torch.full((1,), cap, dtype=torch.int32, device=dev)
    loop = bca.DecodeLoop(q, k, v, kv_len, w.scale, num_splits=num_splits)
    try:
        for L in (cap, 40, 33):
            kv_len.fill_(L)
            torch.cuda.synchronize()
            loop.launch()
            torch.cuda.synchronize()
            for i in range(steps):
                _oracle_check(q[i], k[:L], v[:L], w.scale, loop.out[i], loop.lse[i])
    finally:
        loop.close()
