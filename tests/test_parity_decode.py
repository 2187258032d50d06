"""GPU parity of the split-KV decode step with the oracle, and split-count
invariance (any number of key chunks merges to the same result)."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

from gpu_helpers import TOL_BF16, max_abs

pytestmark = pytest.mark.gpu


def run_decode(w, num_splits=0):
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev).contiguous() for t in (w.q, w.k, w.v))
    o, lse = bca.decode(q, k, v, w.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("P", [1024, 8192])
def test_decode_step_matches_oracle(P):
    w = W.decode_step(P)
    o, lse = run_decode(w)
    O, LSE = oracle.decode(w.q, w.k, w.v, w.scale)
    eo, el = max_abs(o, O), max_abs(lse, LSE)
    print(f"{w.name}: max|dO| = {eo:.3g}, max|dLSE| = {el:.3g}")
    assert eo <= TOL_BF16 and el <= TOL_BF16


@pytest.mark.parametrize("P,B,hq,hkv,d", [
    (0, 32, 32, 8, 128), (68, 16, 4, 4, 128), (1000, 32, 16, 2, 64), (200, 48, 6, 2, 128),
    (64 * 40, 64, 32, 8, 128),
    # two query heads per KV head: a workgroup takes two 32-token sub-tiles,
    # the second here partly past the block's 40 tokens
    (300, 40, 16, 8, 128), (777, 40, 8, 4, 64),
])
def test_decode_edge_shapes(P, B, hq, hkv, d):
    w = W.decode_step(P, block_size=B, hq=hq, hkv=hkv, d=d, seed=5)
    o, lse = run_decode(w)
    O, LSE = oracle.decode(w.q, w.k, w.v, w.scale)
    assert max_abs(o, O) <= TOL_BF16 and max_abs(lse, LSE) <= TOL_BF16


# A workgroup takes the key tiles of its split in rounds of up to five (the
# first round's fifth tile after the query rows): splits of 5 + 1 and 5 + 2
# tiles (129 tiles in 21 splits), 5 + 5 and 5 + 5 + 1 (32 tiles in 3 splits)
# and four rounds (513 tiles in 31 splits, the library's plan), each against
# the oracle.
@pytest.mark.parametrize("P,ns", [(8192, 21), (2048 - 32, 3), (32768, 0)])
def test_decode_multi_round_splits_match_oracle(P, ns):
    w = W.decode_step(P)
    o, lse = run_decode(w, num_splits=ns)
    O, LSE = oracle.decode(w.q, w.k, w.v, w.scale)
    assert max_abs(o, O) <= TOL_BF16 and max_abs(lse, LSE) <= TOL_BF16


def test_split_count_invariance():
    w = W.decode_step(8192)
    ref_o, ref_l = run_decode(w, num_splits=1)
    for ns in (2, 3, 8, 33, 0):
        o, lse = run_decode(w, num_splits=ns)
        # fp32 merge of partials: O agrees to one bf16 rounding step, LSE to fp32 rounding
        assert max_abs(o, ref_o) <= 2 ** -8, ns
        assert max_abs(lse, ref_l) <= 1e-5, ns


def test_decode_is_deterministic():
    w = W.decode_step(8192)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    o1, l1 = bca.decode(q, k, v, w.scale)
    o2, l2 = bca.decode(q, k, v, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_equals_last_block_of_block_causal_forward():
    # The decode entry and the block-causal entry agree on the block's rows.
    P, B = 256, 32
    w = W.decode_step(P, block_size=B, seed=9)
    dev = torch.device("cuda", 0)
    q_full = torch.cat([torch.zeros(P, w.hq, w.d, dtype=torch.bfloat16), w.q]).to(dev)
    k, v = w.k.to(dev), w.v.to(dev)
    cu = torch.tensor([0, P + B], dtype=torch.int32, device=dev)
    o_f, l_f = bca.fwd(q_full, k, v, cu, B, w.scale, P + B)
    o_d, l_d = bca.decode(q_full[P:].contiguous(), k, v, w.scale)
    torch.cuda.synchronize()
    assert max_abs(o_f[P:].float().cpu().numpy(), o_d.float().cpu().numpy()) <= 2 ** -8
    assert max_abs(l_f[:, P:].cpu().numpy(), l_d.cpu().numpy()) <= 1e-5
