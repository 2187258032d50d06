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
