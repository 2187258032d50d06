"""BCA_VALIDATE, BCA_POISON and the staged backward on the GPU.

BCA_VALIDATE=1: a call whose device tables break the header's contract
returns BCA_ERR_SHAPE before anything is enqueued -- the pre-filled outputs
stay untouched -- and a valid call gives the same bits as without the switch.
BCA_POISON=1: NaN-filled workspaces change no output bit (every workspace word
a kernel reads was written by a kernel of the same call).  The backward run as
stages 1, 3, 2 equals the one-call backward bit for bit.
"""
import os

import numpy as np
import pytest
import torch

from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd import workloads as W

from gpu_helpers import device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture
def env(monkeypatch):
    def set_(name, on):
        if on:
            monkeypatch.setenv(name, "1")
        else:
            monkeypatch.delenv(name, raising=False)
    return set_


def small():
    return W.packed("validate", "staircase_bwd", 77, [96 + 3 * 32, 64 + 2 * 32, 100], [3, 2, 0],
                    8, 2, 128, 32, "bf16", with_do=True)


def i32(x, dev):
    return torch.tensor(x, dtype=torch.int32, device=dev)


def test_validation_rejects_bad_tables_before_any_launch(env):
    w = small()
    q, k, v, cu, sc, do = device_inputs(w)
    dev = q.device
    env("BCA_VALIDATE", True)
    lens = np.diff(w.cu_seqlens)
    bad = {
        "cu[0] != 0": (i32([4] + list(w.cu_seqlens[1:]), dev), sc, w.max_seqlen),
        "decreasing cu": (i32([0, 200, 150, w.total], dev), sc, w.max_seqlen),
        "cu[nseq] != total": (i32(list(w.cu_seqlens[:-1]) + [w.total - 1], dev), sc,
                              w.max_seqlen),
        "max_seqlen too small": (cu, sc, int(lens.max()) - 1),
        "too many copies": (cu, i32([3, 9, 0], dev), w.max_seqlen),
        "negative copies": (cu, i32([3, -1, 0], dev), w.max_seqlen),
        "prefix not a multiple of B": (cu, i32([0, 0, 1], dev), w.max_seqlen),
    }
    for name, (cu_b, sc_b, ms) in bad.items():
        o = torch.full_like(q, 7.0)
        lse = torch.full((w.hq, w.total), 7.0, device=dev)
        with pytest.raises(bca.BcaError) as e:
            bca.staircase_fwd(q, k, v, cu_b, sc_b, w.block_size, w.scale, ms, out=o, lse=lse)
        assert e.value.status == 2 and "validation" in str(e.value), (name, str(e.value))
        with pytest.raises(bca.BcaError) as e:
            bca.staircase_bwd(q, k, v, o, lse, do, cu_b, sc_b, w.block_size, w.scale, ms)
        assert e.value.status == 2, name
        torch.cuda.synchronize()
        assert bool((o == 7.0).all()) and bool((lse == 7.0).all()), name  # nothing ran


def test_validation_rejects_bad_group_tables(env):
    w = W.general_staircase("validate_groups", 5, 2, 32, 2, 4, 1, 2, 4, 2, 128, "bf16")
    q, k, v, cu, _, _ = device_inputs(w)
    dev = q.device
    gs, gp, gc = (torch.from_numpy(x).to(dev) for x in w.group_table())
    env("BCA_VALIDATE", True)
    o, lse = bca.staircase_groups_fwd(q, k, v, cu, gs, gp, gc, w.block_size, w.scale, w.max_seqlen)
    torch.cuda.synchronize()
    bad = {
        "pe not a multiple of B": (gs, gp + 1, gc),
        "pe beyond the prefix": (gs, gp + 10 * w.block_size, gc),
        "negative copies": (gs, gp, gc - 5),
        "group_start decreasing": (gs.flip(0), gp, gc),
    }
    for name, (a, b, c) in bad.items():
        with pytest.raises(bca.BcaError) as e:
            bca.staircase_groups_fwd(q, k, v, cu, a.contiguous(), b.contiguous(), c.contiguous(),
                                     w.block_size, w.scale, w.max_seqlen)
        assert e.value.status == 2 and "validation" in str(e.value), (name, str(e.value))


def test_validation_passes_valid_calls_unchanged(env):
    w = small()
    q, k, v, cu, sc, do = device_inputs(w)
    env("BCA_VALIDATE", False)
    o1, l1 = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    g1 = bca.staircase_bwd(q, k, v, o1, l1, do, cu, sc, w.block_size, w.scale, w.max_seqlen)
    env("BCA_VALIDATE", True)
    o2, l2 = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    g2 = bca.staircase_bwd(q, k, v, o2, l2, do, cu, sc, w.block_size, w.scale, w.max_seqlen)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_poisoned_workspaces_change_nothing(env):
    w = small()
    q, k, v, cu, sc, do = device_inputs(w)
    o, lse = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    env("BCA_POISON", False)
    g1 = bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, w.block_size, w.scale, w.max_seqlen)
    wd = W.decode_step(1024)
    qd, kd, vd = (t.to(q.device) for t in (wd.q, wd.k, wd.v))
    d1 = bca.decode(qd, kd, vd, wd.scale)
    env("BCA_POISON", True)
    g2 = bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, w.block_size, w.scale, w.max_seqlen)
    d2 = bca.decode(qd, kd, vd, wd.scale)
    torch.cuda.synchronize()
    for a, b in zip(g1 + d1, g2 + d2):
        assert torch.equal(a, b)


def test_staged_backward_equals_one_call():
    w = small()
    q, k, v, cu, sc, do = device_inputs(w)
    o, lse = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    full = bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, w.block_size, w.scale, w.max_seqlen)
    ws = torch.empty(bca.staircase_bwd_workspace(w.total, w.hq, w.hkv, w.d), dtype=torch.uint8,
                     device=q.device)
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in full)
    for stage in (1, 3, 2):
        bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, w.block_size, w.scale, w.max_seqlen,
                          workspace=ws, dq=dq, dk=dk, dv=dv, stage=stage)
    torch.cuda.synchronize()
    for a, b in zip(full, (dq, dk, dv)):
        assert torch.equal(a, b)
