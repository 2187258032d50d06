"""The Python binding's own argument checks (no GPU needed).

Every wrapper checks shapes and dtypes of all its tensors -- inputs, caller
supplied outputs and the workspace -- before it touches the device or the
library, because the kernels index with q's dtype and head_dim: a mismatched
tensor would be read or written out of bounds.  These run on CPU tensors: a
shape or dtype error must be raised before the "tensors must live on the GPU"
check is reached.
"""
import pytest
import torch

from block_diffusion_lm_causal_amd import bca

BF, F32 = torch.bfloat16, torch.float32


def packed(total=64, hq=8, hkv=2, d=128, dt=BF):
    q = torch.zeros(total, hq, d, dtype=dt)
    k = torch.zeros(total, hkv, d, dtype=dt)
    v = torch.zeros(total, hkv, d, dtype=dt)
    cu = torch.tensor([0, total], dtype=torch.int32)
    return q, k, v, cu


def expect(status, fn, *a, **kw):
    with pytest.raises(bca.BcaError) as e:
        fn(*a, **kw)
    assert e.value.status == status, str(e.value)
    assert "GPU" not in str(e.value), str(e.value)
    return str(e.value)


def test_forward_checks():
    q, k, v, cu = packed()
    for fn in (lambda **kw: bca.fwd(kw.pop("q", q), kw.pop("k", k), kw.pop("v", v), cu, 32, **kw),
               lambda **kw: bca.staircase_fwd(kw.pop("q", q), kw.pop("k", k), kw.pop("v", v), cu,
                                              None, 32, **kw)):
        assert "k must be" in expect(3, fn, k=k.float())            # k dtype differs from q
        assert "v must have" in expect(2, fn, v=v[:, :, :64])        # head_dim differs
        assert "k must have" in expect(2, fn, k=k[:32])              # token count differs
        expect(3, fn, q=q.half(), k=k.half(), v=v.half())           # unsupported dtype
        expect(2, fn, q=q[0])                                       # not 3-D
        assert "out" in expect(2, fn, out=torch.zeros(64, 8, 64, dtype=BF))
        assert "out" in expect(3, fn, out=torch.zeros(64, 8, 128, dtype=F32))
        assert "lse" in expect(2, fn, lse=torch.zeros(64, 8))
        assert "lse" in expect(3, fn, lse=torch.zeros(8, 64, dtype=BF))
    bad_sc = torch.zeros(2, dtype=torch.int32)
    assert "s_copies" in expect(2, bca.staircase_fwd, q, k, v, cu, bad_sc, 32)
    expect(2, bca.fwd, q, k, v, cu.long(), 32)


def test_backward_checks():
    q, k, v, cu = packed()
    o, do, lse = torch.zeros_like(q), torch.zeros_like(q), torch.zeros(8, 64)

    def call(**kw):
        a = dict(q=q, k=k, v=v, o=o, lse=lse, dout=do)
        a.update({n: kw.pop(n) for n in list(kw) if n in a})
        return bca.staircase_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], cu, None,
                                 32, **kw)
    expect(3, call, q=q.float(), k=k.float(), v=v.float())         # backward is bf16 only
    assert "o must" in expect(3, call, o=o.float())
    assert "dout must" in expect(2, call, dout=do[:, :4])
    assert "lse must" in expect(2, call, lse=lse.t().contiguous())
    assert "dq must" in expect(2, call, dq=torch.zeros(64, 8, 64, dtype=BF))
    assert "dk must" in expect(2, call, dk=torch.zeros_like(q))
    assert "dv must" in expect(3, call, dv=torch.zeros_like(v, dtype=F32))
    assert "workspace" in expect(2, call, workspace=torch.zeros(4, 4, dtype=torch.uint8))
    assert "s_copies" in expect(2, bca.staircase_bwd, q, k, v, o, lse, do, cu,
                                torch.zeros(3, dtype=torch.int32), 32)


def test_decode_checks():
    q = torch.zeros(32, 8, 128, dtype=BF)
    k = torch.zeros(288, 2, 128, dtype=BF)
    expect(3, bca.decode, q.float(), k, k)
    assert "k must be" in expect(3, bca.decode, q, k.float(), k)
    assert "v must have" in expect(2, bca.decode, q, k, k[:, :, :64])   # head_dim of q is 128
    assert "out" in expect(2, bca.decode, q, k, k, out=torch.zeros(32, 8, 64, dtype=BF))
    assert "lse" in expect(2, bca.decode, q, k, k, lse=torch.zeros(32, 8))
    k8 = torch.zeros(288, 2, 128, dtype=torch.uint8)
    assert "k8" in expect(3, bca.decode_fp8, q, k.float(), k8, 1.0, 1.0)
    assert "v8" in expect(2, bca.decode_fp8, q, k8, k8[:, :, :64], 1.0, 1.0)
    expect(3, bca.decode_fp8, q.float(), k8, k8, 1.0, 1.0)
    assert "k must be" in expect(3, bca.DecodeGraph, q, k.float(), k, 4)


def test_decode_loop_checks():
    q = torch.zeros(4, 32, 8, 128, dtype=BF)
    k = torch.zeros(288, 2, 128, dtype=BF)
    n = torch.zeros(1, dtype=torch.int32)
    expect(2, bca.DecodeLoop, q[0], k, k, n)                           # q needs a step axis
    expect(3, bca.DecodeLoop, q.float(), k, k, n)
    assert "v must have" in expect(2, bca.DecodeLoop, q, k, k[:, :, :64], n)
    assert "out" in expect(2, bca.DecodeLoop, q, k, k, n, out=torch.zeros(32, 8, 128, dtype=BF))
    assert "lse" in expect(2, bca.DecodeLoop, q, k, k, n, lse=torch.zeros(8, 32))
    assert "kv_len_dev" in expect(2, bca.DecodeLoop, q, k, k, n.long())
    assert "steps_dev" in expect(2, bca.DecodeLoop, q, k, k, n, steps_dev=n.float())
