"""The C ABI without a GPU: exported symbols and host-side argument checks.

Every call here fails validation (or has nothing to do) before the library
touches the HIP runtime, so these run on a machine with no GPU.  The fake
device pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from block_diffusion_lm_causal_amd import bca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bca.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bca.LIB_PATH):
        pytest.skip("libbca.so not built")
    return bca.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bca_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(bca.EXPORTS)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert bca.abi_version() == 1
    assert L.bca_status_string(OK) == b"ok"
    assert L.bca_status_string(WS) == b"workspace too small"
    assert L.bca_status_string(99) == b"unknown status"


def fwd(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, s=None, nseq=1, max_seqlen=64,
             total=64, hq=32, hkv=8, d=128, B=32, scale=0.088, dt=BF16)
    a.update(kw)
    return L.bca_staircase_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["s"],
                               a["nseq"], a["max_seqlen"], a["total"], a["hq"], a["hkv"], a["d"],
                               a["B"], a["scale"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(hq=6, hkv=4), SHAPE), (dict(hkv=0), SHAPE),
    (dict(B=0), SHAPE), (dict(B=-3), SHAPE), (dict(nseq=-1), SHAPE), (dict(total=-5), SHAPE),
    (dict(max_seqlen=0), SHAPE), (dict(q=None), NULL), (dict(lse=None), NULL),
    (dict(cu=None), NULL), (dict(dt=7), DTYPE), (dict(scale=float("nan")), SHAPE),
    (dict(q=ctypes.c_void_p((1 << 20) + 8)), SHAPE),
])
def test_forward_rejects_bad_arguments(L, kw, status):
    assert fwd(L, **kw) == status
    assert L.bca_last_error() != b""


def test_forward_with_nothing_to_do_is_ok(L):
    # No segments, or no tokens: nothing is enqueued and NULL data is fine.
    assert fwd(L, nseq=0, q=None, k=None, v=None, o=None, lse=None, cu=None) == OK
    assert fwd(L, total=0, q=None, k=None, v=None, o=None, lse=None) == OK
    assert L.bca_last_error() == b""


def test_block_causal_entry_validates_too(L):
    st = L.bca_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 64, 32, 8, 100, 32, 0.1, BF16, None)
    assert st == UNSUP


def bwd(L, ws_bytes, **kw):
    a = dict(dt=BF16, ws=FAKE, dout=FAKE, hq=32, hkv=8, d=128, total=1000)
    a.update(kw)
    return L.bca_staircase_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, a["dout"], FAKE, FAKE, FAKE, FAKE,
                               None, 1, 1000, a["total"], a["hq"], a["hkv"], a["d"], 32, 0.1,
                               a["dt"], a["ws"], ws_bytes, None)


def test_backward_workspace_and_checks(L):
    need = L.bca_staircase_bwd_workspace(1000, 32, 8, 128)
    assert need >= 2 * 32 * 1000 * 4  # delta and LSE * log2(e)
    assert bwd(L, need - 1) == WS
    assert bwd(L, need, ws=None) == WS
    assert bwd(L, need, dt=F32) == DTYPE
    assert bwd(L, need, dout=None) == NULL
    assert bwd(L, need, d=80) == UNSUP
    assert L.bca_staircase_bwd_workspace(-1, 32, 8, 128) == 0


def dec(L, ws, ws_bytes, **kw):
    a = dict(q_len=32, kv_len=1056, hq=32, hkv=8, d=128, dt=BF16, ns=0, q=FAKE)
    a.update(kw)
    return L.bca_decode(a["q"], FAKE, FAKE, FAKE, FAKE, a["q_len"], a["kv_len"], a["hq"], a["hkv"],
                        a["d"], 0.088, a["dt"], a["ns"], ws, ws_bytes, None)


def test_decode_workspace_and_checks(L):
    need = L.bca_decode_workspace(32, 1056, 32, 8, 128, 0)
    assert need > 0
    # one split writes O directly: no workspace
    assert L.bca_decode_workspace(32, 1056, 32, 8, 128, 1) == 0
    assert L.bca_decode_workspace(32, 1056, 32, 8, 100, 0) == 0
    more = L.bca_decode_workspace(32, 8224, 32, 8, 128, 8)
    assert more == 8 * 32 * 32 * 128 * 2 + 8 * 32 * 32 * 4  # bf16 partial O, float32 LSE
    assert dec(L, FAKE, need - 1) == WS
    assert dec(L, None, need) == WS
    assert dec(L, FAKE, need, kv_len=16) == SHAPE       # kv_len < q_len
    assert dec(L, FAKE, need, q_len=0) == SHAPE
    assert dec(L, FAKE, need, hq=12) == SHAPE
    assert dec(L, FAKE, need, d=32) == UNSUP
    assert dec(L, FAKE, need, dt=F32) == DTYPE
    assert dec(L, FAKE, need, ns=-2) == SHAPE
    assert dec(L, FAKE, need, ns=257) == SHAPE
    assert dec(L, FAKE, need, q=None) == NULL


def test_binding_requires_gpu_tensors():
    import torch
    if not os.path.exists(bca.LIB_PATH):
        pytest.skip("libbca.so not built")
    q = torch.zeros(4, 1, 64)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(bca.BcaError):
        bca.fwd(q, q, q, cu, 2)


def test_decode_graph_checks(L):
    h = ctypes.c_void_p()
    need = L.bca_decode_workspace(32, 1056, 32, 8, 128, 0)

    def create(steps=4, dt=BF16, ws=FAKE, handle=ctypes.byref(h), q=FAKE):
        return L.bca_decode_graph_create(q, FAKE, FAKE, FAKE, FAKE, 32, 1056, 32, 8, 128, 0.088,
                                         dt, 0, ws, need, steps, handle)
    assert create(steps=0) == SHAPE and not h.value
    assert create(steps=5000) == SHAPE
    assert create(dt=F32) == DTYPE
    assert create(ws=None) == WS
    assert create(q=None) == NULL
    assert create(handle=None) == NULL
    L.bca_decode_graph_destroy(None)  # no-op
    assert L.bca_decode_graph_launch(None, None) == NULL


def test_decode_loop_checks(L):
    h = ctypes.c_void_p()
    need = L.bca_decode_workspace(32, 2080, 32, 8, 128, 0)

    def create(steps=4, lenp=FAKE, stepsp=None, cap=2080, ws=FAKE, handle=ctypes.byref(h)):
        return L.bca_decode_loop_create(FAKE, FAKE, FAKE, FAKE, FAKE, lenp, stepsp, 32, cap, 32,
                                        8, 128, 0.088, BF16, 0, ws, need, steps, handle)
    assert create(lenp=None) == NULL and not h.value
    assert create(lenp=ctypes.c_void_p((1 << 20) + 2)) == SHAPE   # int32 alignment
    assert create(stepsp=ctypes.c_void_p((1 << 20) + 2)) == SHAPE
    assert create(steps=0) == SHAPE
    assert create(steps=5000) == SHAPE
    assert create(cap=16) == SHAPE               # capacity below q_len
    assert create(ws=None) == WS
    assert create(handle=None) == NULL


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf")])
def test_scale_must_be_positive_and_finite(L, scale):
    # The kernels take the row maximum of the raw scores before scaling, which
    # is the maximum of the scaled scores only for a positive scale.
    assert fwd(L, scale=scale) == SHAPE
    assert L.bca_staircase_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               1, 64, 64, 32, 8, 128, 32, scale, BF16, FAKE, 1 << 30,
                               None) == SHAPE
    assert L.bca_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 32, 1056, 32, 8, 128, scale, BF16, 0, FAKE,
                        1 << 30, None) == SHAPE
    assert b"scale" in L.bca_last_error()


def stage_call(L, stage, **kw):
    a = dict(ws=FAKE, nseq=1)
    a.update(kw)
    return L.bca_staircase_bwd_stage(stage, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, None, a["nseq"], 1000, 1000, 32, 8, 128, 32, 0.1, BF16,
                                     a["ws"], 1 << 30, None)


def test_backward_stage_checks(L):
    for bad in (-1, 4, 99):
        assert stage_call(L, bad) == SHAPE
        assert b"stage" in L.bca_last_error()
    for stage in (0, 1, 2, 3):  # valid stages still check the workspace, before any launch
        assert stage_call(L, stage, ws=None) == WS
        assert stage_call(L, stage, nseq=0) == OK


def test_status_strings_cover_every_code(L):
    names = {L.bca_status_string(c) for c in range(8)}
    assert len(names) == 8 and b"unknown status" not in names
    assert L.bca_status_string(7) == b"host memory exhausted"
    assert L.bca_status_string(8) == b"unknown status"


def test_noalloc_decode_checks_before_touching_the_gpu(L):
    def call(**kw):
        a = dict(q=FAKE, q_len=32, kv_len=8224, hq=32, d=128, ns=0, dt=BF16)
        a.update(kw)
        return L.bca_decode_noalloc(a["q"], FAKE, FAKE, FAKE, FAKE, a["q_len"], a["kv_len"],
                                    a["hq"], 8, a["d"], 0.088, a["dt"], a["ns"], None)
    assert call(ns=256) == WS                       # 64 MiB of partials > 32 MiB held
    assert b"scratch" in L.bca_last_error()
    assert call(q_len=0) == SHAPE
    assert call(d=96) == UNSUP
    assert call(dt=F32) == DTYPE
