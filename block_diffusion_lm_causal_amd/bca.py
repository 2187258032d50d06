"""Python binding of libbca.so (ctypes): argument marshalling only.

Every step of the attention runs in the library's HIP kernels; this module
checks tensor placement, allocates outputs with torch (device memory and
streams are all torch provides here) and passes raw pointers and sizes to the
C ABI declared in include/bca.h.  There is no fallback: if the library is
missing or a call fails, a ``BcaError`` is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbca.so")

BCA_F32 = 0
BCA_BF16 = 1

# Every symbol include/bca.h declares.
EXPORTS = (
    "bca_abi_version", "bca_status_string", "bca_last_error", "bca_fwd", "bca_staircase_fwd",
    "bca_staircase_bwd_workspace", "bca_staircase_bwd", "bca_decode_workspace", "bca_decode",
    "bca_decode_graph_create", "bca_decode_graph_launch", "bca_decode_graph_destroy",
    "bca_trajectory_cost", "bca_pack_balanced", "bca_pack_last_error",
    "bca_staircase_groups_fwd", "bca_staircase_groups_bwd", "bca_decode_fp8",
    "bca_staircase_bwd_stage", "bca_decode_noalloc", "bca_trajectory_cost_groups",
    "bca_pack_balanced_groups", "bca_decode_loop_create",
)


class BcaError(RuntimeError):
    """A libbca call returned a non-zero status, or the library is unavailable."""

    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func}: status {status}: {message}")
        self.func = func
        self.status = status


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_S = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libbca.so once (raises BcaError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise BcaError("load", -1, f"{LIB_PATH} is missing; build it with "
                       "`python -m block_diffusion_lm_causal_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.bca_abi_version.restype = _I
    L.bca_abi_version.argtypes = []
    L.bca_status_string.restype = ctypes.c_char_p
    L.bca_status_string.argtypes = [_I]
    L.bca_last_error.restype = ctypes.c_char_p
    L.bca_last_error.argtypes = []
    L.bca_fwd.restype = _I
    L.bca_fwd.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]
    L.bca_staircase_fwd.restype = _I
    L.bca_staircase_fwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                    _I, _P]
    L.bca_staircase_bwd_workspace.restype = _S
    L.bca_staircase_bwd_workspace.argtypes = [_I, _I, _I, _I]
    L.bca_staircase_bwd.restype = _I
    L.bca_staircase_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                    _I, _I, _I, _F, _I, _P, _S, _P]
    L.bca_staircase_bwd_stage.restype = _I
    L.bca_staircase_bwd_stage.argtypes = [_I] + L.bca_staircase_bwd.argtypes
    L.bca_decode_workspace.restype = _S
    L.bca_decode_workspace.argtypes = [_I, _I, _I, _I, _I, _I]
    L.bca_decode.restype = _I
    L.bca_decode.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P]
    L.bca_decode_noalloc.restype = _I
    L.bca_decode_noalloc.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]
    L.bca_decode_graph_create.restype = _I
    L.bca_decode_graph_create.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P,
                                          _S, _I, ctypes.POINTER(_P)]
    L.bca_decode_loop_create.restype = _I
    L.bca_decode_loop_create.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I,
                                         _I, _P, _S, _I, ctypes.POINTER(_P)]
    L.bca_decode_graph_launch.restype = _I
    L.bca_decode_graph_launch.argtypes = [_P, _P]
    L.bca_decode_graph_destroy.restype = None
    L.bca_decode_graph_destroy.argtypes = [_P]
    L.bca_staircase_groups_fwd.restype = _I
    L.bca_staircase_groups_fwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                           _I, _I, _I, _F, _I, _P]
    L.bca_staircase_groups_bwd.restype = _I
    L.bca_staircase_groups_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _S, _P]
    L.bca_decode_fp8.restype = _I
    L.bca_decode_fp8.argtypes = [_P, _P, _P, _F, _F, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _S,
                                 _P]
    L.bca_trajectory_cost.restype = ctypes.c_int64
    L.bca_trajectory_cost.argtypes = [_I, _I, _I]
    L.bca_pack_balanced.restype = _I
    L.bca_pack_balanced.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _P]
    L.bca_trajectory_cost_groups.restype = ctypes.c_int64
    L.bca_trajectory_cost_groups.argtypes = [_I, _P, _P, _I, _I]
    L.bca_pack_balanced_groups.restype = _I
    L.bca_pack_balanced_groups.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P]
    L.bca_pack_last_error.restype = ctypes.c_char_p
    L.bca_pack_last_error.argtypes = []
    _lib = L
    return L


def abi_version() -> int:
    return int(lib().bca_abi_version())


def _check(func: str, status: int) -> None:
    if status != 0:
        L = lib()
        msg = L.bca_last_error().decode() or L.bca_status_string(status).decode()
        raise BcaError(func, status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on(device: torch.device, fn, *args):
    """Call a library entry point with the tensors' device current (the C ABI
    takes the calling thread's current device to be the device of its
    pointers and stream, as HIP does)."""
    with torch.cuda.device(device):
        return fn(*args)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BCA_BF16
    if t.dtype == torch.float32:
        return BCA_F32
    raise BcaError("dtype", 3, f"unsupported tensor dtype {t.dtype}")


def _need_gpu(*ts: Optional[torch.Tensor]) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise BcaError("args", 2, "tensors must live on the GPU")
        if not t.is_contiguous():
            raise BcaError("args", 2, "tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise BcaError("args", 2, "tensors must share one device")
    return dev


def _expect(func: str, t: Optional[torch.Tensor], name: str, shape, dtype) -> None:
    """Raise BcaError unless tensor t (if given) has this shape and dtype."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise BcaError(func, 2, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise BcaError(func, 3, f"{name} must be {dtype}, got {t.dtype}")


def _packed_shapes(func: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   dtypes=(torch.bfloat16, torch.float32)):
    """(total, hq, hkv, d) of packed inputs, after checking that q is
    [total, hq, d] and k, v are [total, hkv, d] of q's dtype."""
    if q.dim() != 3 or k.dim() != 3:
        raise BcaError(func, 2, "q must be [total, hq, d] and k, v [total, hkv, d]")
    if q.dtype not in dtypes:
        raise BcaError(func, 3, f"q must be one of {dtypes}, got {q.dtype}")
    total, hq, d = q.shape
    hkv = k.shape[1]
    _expect(func, k, "k", (total, hkv, d), q.dtype)
    _expect(func, v, "v", (total, hkv, d), q.dtype)
    return total, hq, hkv, d


def _seq_args(cu_seqlens: torch.Tensor, max_seqlen: Optional[int]):
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise BcaError("args", 2, "cu_seqlens must be a 1-D int32 tensor of nseq + 1 entries")
    nseq = cu_seqlens.numel() - 1
    if max_seqlen is None:  # convenience: one device-to-host read
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if nseq > 0 else 0
    return nseq, int(max_seqlen)


def staircase_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                  s_copies: Optional[torch.Tensor], block_size: int,
                  scale: Optional[float] = None, max_seqlen: Optional[int] = None,
                  out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Staircase (or, with s_copies=None, block-causal) forward -> (O, LSE).

    q [total, hq, d], k/v [total, hkv, d] (bf16 or float32), cu_seqlens int32
    [nseq + 1] and s_copies int32 [nseq] on the same GPU.  LSE is [hq, total]
    float32 (natural log).
    """
    total, hq, hkv, d = _packed_shapes("staircase_fwd", q, k, v)
    _expect("staircase_fwd", out, "out", (total, hq, d), q.dtype)
    _expect("staircase_fwd", lse, "lse", (hq, total), torch.float32)
    nseq, max_seqlen = _seq_args(cu_seqlens, max_seqlen)
    _expect("staircase_fwd", s_copies, "s_copies", (nseq,), torch.int32)
    dev = _need_gpu(q, k, v, cu_seqlens, s_copies, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, total), dtype=torch.float32, device=dev)
    st = _on(dev, lib().bca_staircase_fwd,
             _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), _ptr(s_copies),
             nseq, max_seqlen, total, hq, hkv, d, int(block_size), scale, _dtype_code(q),
             _stream(dev))
    _check("bca_staircase_fwd", st)
    return out, lse


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
        block_size: int, scale: Optional[float] = None, max_seqlen: Optional[int] = None,
        out: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block-causal forward over packed sequences -> (O, LSE); see staircase_fwd."""
    total, hq, hkv, d = _packed_shapes("fwd", q, k, v)
    _expect("fwd", out, "out", (total, hq, d), q.dtype)
    _expect("fwd", lse, "lse", (hq, total), torch.float32)
    nseq, max_seqlen = _seq_args(cu_seqlens, max_seqlen)
    dev = _need_gpu(q, k, v, cu_seqlens, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, total), dtype=torch.float32, device=dev)
    st = _on(dev, lib().bca_fwd,
             _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), nseq, max_seqlen,
             total, hq, hkv, d, int(block_size), scale, _dtype_code(q), _stream(dev))
    _check("bca_fwd", st)
    return out, lse


def _groups_args(func, group_start, group_pe, group_copies, nseq):
    for t, name in ((group_start, "group_start"), (group_pe, "group_pe"),
                    (group_copies, "group_copies")):
        if t is None or t.dtype != torch.int32:
            raise BcaError(func, 2, f"{name} must be an int32 tensor")
    if (group_start.dim() != 1 or group_pe.dim() != 1 or group_copies.dim() != 1
            or group_start.numel() != nseq + 1 or group_pe.numel() != group_copies.numel()):
        raise BcaError(func, 2, "group_start must be [nseq + 1]; group_pe and group_copies "
                                "must have one entry per group")


def staircase_groups_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         cu_seqlens: torch.Tensor, group_start: torch.Tensor,
                         group_pe: torch.Tensor, group_copies: torch.Tensor, block_size: int,
                         scale: Optional[float] = None, max_seqlen: Optional[int] = None,
                         out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """General trajectory staircase forward -> (O, LSE): copy groups per segment,
    group g's copies seeing the clean keys [0, group_pe[g])."""
    total, hq, hkv, d = _packed_shapes("staircase_groups_fwd", q, k, v)
    _expect("staircase_groups_fwd", out, "out", (total, hq, d), q.dtype)
    _expect("staircase_groups_fwd", lse, "lse", (hq, total), torch.float32)
    nseq, max_seqlen = _seq_args(cu_seqlens, max_seqlen)
    _groups_args("staircase_groups_fwd", group_start, group_pe, group_copies, nseq)
    dev = _need_gpu(q, k, v, cu_seqlens, group_start, group_pe, group_copies, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, total), dtype=torch.float32, device=dev)
    st = _on(dev, lib().bca_staircase_groups_fwd,
             _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), _ptr(group_start),
             _ptr(group_pe), _ptr(group_copies), nseq, max_seqlen, total, hq, hkv, d,
             int(block_size), scale, _dtype_code(q), _stream(dev))
    _check("bca_staircase_groups_fwd", st)
    return out, lse


def _bwd_checks(func: str, q, k, v, o, lse, dout, dq, dk, dv, workspace):
    """Shapes and dtypes of a backward call: everything bf16, o/dout/dq like q,
    dk/dv like k, lse float32 [hq, total], the workspace a 1-D byte buffer."""
    total, hq, hkv, d = _packed_shapes(func, q, k, v, dtypes=(torch.bfloat16,))
    for t, name in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _expect(func, t, name, (total, hq, d), torch.bfloat16)
    for t, name in ((dk, "dk"), (dv, "dv")):
        _expect(func, t, name, (total, hkv, d), torch.bfloat16)
    _expect(func, lse, "lse", (hq, total), torch.float32)
    if workspace is not None and workspace.dim() != 1:
        raise BcaError(func, 2, "workspace must be a 1-D buffer")
    return total, hq, hkv, d


def staircase_groups_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                         lse: torch.Tensor, dout: torch.Tensor, cu_seqlens: torch.Tensor,
                         group_start: torch.Tensor, group_pe: torch.Tensor,
                         group_copies: torch.Tensor, block_size: int,
                         scale: Optional[float] = None, max_seqlen: Optional[int] = None,
                         workspace: Optional[torch.Tensor] = None,
                         dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                         dv: Optional[torch.Tensor] = None):
    """General trajectory staircase backward -> (dQ, dK, dV), bf16."""
    total, hq, hkv, d = _bwd_checks("staircase_groups_bwd", q, k, v, o, lse, dout, dq, dk, dv,
                                    workspace)
    dev = _need_gpu(q, k, v, o, lse, dout, cu_seqlens, group_start, group_pe, group_copies,
                    workspace, dq, dk, dv)
    nseq, max_seqlen = _seq_args(cu_seqlens, max_seqlen)
    _groups_args("staircase_groups_bwd", group_start, group_pe, group_copies, nseq)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = staircase_bwd_workspace(total, hq, hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    st = _on(dev, lib().bca_staircase_groups_bwd,
             _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
             _ptr(dv), _ptr(cu_seqlens), _ptr(group_start), _ptr(group_pe), _ptr(group_copies),
             nseq, max_seqlen, total, hq, hkv, d, int(block_size), scale, _dtype_code(q),
             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check("bca_staircase_groups_bwd", st)
    return dq, dk, dv


def staircase_bwd_workspace(total: int, hq: int, hkv: int, d: int) -> int:
    return int(lib().bca_staircase_bwd_workspace(total, hq, hkv, d))


def staircase_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                  lse: torch.Tensor, dout: torch.Tensor, cu_seqlens: torch.Tensor,
                  s_copies: Optional[torch.Tensor], block_size: int,
                  scale: Optional[float] = None, max_seqlen: Optional[int] = None,
                  workspace: Optional[torch.Tensor] = None,
                  dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                  dv: Optional[torch.Tensor] = None, stage: int = 0):
    """Backward -> (dQ, dK, dV), bf16.  o and lse come from staircase_fwd.

    ``stage`` selects bca_staircase_bwd_stage: 0 runs everything; 1 the row
    terms, 2 dK/dV and 3 dQ (2 and 3 need the workspace stage 1 filled)."""
    total, hq, hkv, d = _bwd_checks("staircase_bwd", q, k, v, o, lse, dout, dq, dk, dv,
                                    workspace)
    nseq = cu_seqlens.numel() - 1
    _expect("staircase_bwd", s_copies, "s_copies", (nseq,), torch.int32)
    dev = _need_gpu(q, k, v, o, lse, dout, cu_seqlens, s_copies, workspace, dq, dk, dv)
    nseq, max_seqlen = _seq_args(cu_seqlens, max_seqlen)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = staircase_bwd_workspace(total, hq, hkv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _on(dev, lib().bca_staircase_bwd_stage,
             int(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
             _ptr(dk), _ptr(dv), _ptr(cu_seqlens), _ptr(s_copies), nseq, max_seqlen, total, hq, hkv,
             d, int(block_size), scale, _dtype_code(q), _ptr(workspace), ws_bytes, _stream(dev))
    _check("bca_staircase_bwd_stage", st)
    return dq, dk, dv


def decode_workspace(q_len: int, kv_len: int, hq: int, hkv: int, d: int,
                     num_splits: int = 0) -> int:
    return int(lib().bca_decode_workspace(q_len, kv_len, hq, hkv, d, num_splits))


def _decode_shapes(func: str, q, k, v, out, lse, kv_dtype):
    """(q_len, hq, kv_len, hkv, d) of a decode call after checking q [q_len,
    hq, d] bf16, k/v [kv_len, hkv, d] of kv_dtype (None: any one-byte type),
    out like q and lse float32 [hq, q_len]."""
    if q.dim() != 3 or k.dim() != 3:
        raise BcaError(func, 2, "q must be [q_len, hq, d] and k, v [kv_len, hkv, d]")
    if q.dtype != torch.bfloat16:
        raise BcaError(func, 3, f"q must be torch.bfloat16, got {q.dtype}")
    q_len, hq, d = q.shape
    kv_len, hkv = k.shape[0], k.shape[1]
    if kv_dtype is None:
        for t, name in ((k, "k8"), (v, "v8")):
            if t.element_size() != 1:
                raise BcaError(func, 3, f"{name} must hold one byte per element")
        _expect(func, k, "k8", (kv_len, hkv, d), None)
        _expect(func, v, "v8", (kv_len, hkv, d), None)
    else:
        _expect(func, k, "k", (kv_len, hkv, d), kv_dtype)
        _expect(func, v, "v", (kv_len, hkv, d), kv_dtype)
    _expect(func, out, "out", (q_len, hq, d), torch.bfloat16)
    _expect(func, lse, "lse", (hq, q_len), torch.float32)
    return q_len, hq, kv_len, hkv, d


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
           num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode step -> (O [q_len, hq, d], LSE [hq, q_len]); k/v hold prefix + block rows."""
    q_len, hq, kv_len, hkv, d = _decode_shapes("decode", q, k, v, out, lse, torch.bfloat16)
    dev = _need_gpu(q, k, v, workspace, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = decode_workspace(q_len, kv_len, hq, hkv, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, q_len), dtype=torch.float32, device=dev)
    st = _on(dev, lib().bca_decode,
             _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), q_len, kv_len, hq, hkv, d, scale,
             _dtype_code(q), int(num_splits), _ptr(workspace), ws_bytes, _stream(dev))
    _check("bca_decode", st)
    return out, lse


def decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   scale: Optional[float] = None, num_splits: int = 0,
                   out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode step with the library's own per-GPU scratch (bca_decode_noalloc):
    no workspace is allocated; pass ``out`` and ``lse`` to allocate nothing at
    all.  Calls that overlap on one GPU race on the shared scratch."""
    q_len, hq, kv_len, hkv, d = _decode_shapes("decode_noalloc", q, k, v, out, lse,
                                               torch.bfloat16)
    dev = _need_gpu(q, k, v, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, q_len), dtype=torch.float32, device=dev)
    st = _on(dev, lib().bca_decode_noalloc,
             _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), q_len, kv_len, hq, hkv, d, scale,
             _dtype_code(q), int(num_splits), _stream(dev))
    _check("bca_decode_noalloc", st)
    return out, lse


def decode_fp8(q: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, k_scale: float,
               v_scale: float, scale: Optional[float] = None, num_splits: int = 0,
               workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode step against an FP8 E4M3 cache -> (O bf16 [q_len, hq, d], LSE [hq, q_len]).

    k8/v8 are [kv_len, hkv, d] uint8 (or float8_e4m3fn) holding K / k_scale
    and V / v_scale.
    """
    q_len, hq, kv_len, hkv, d = _decode_shapes("decode_fp8", q, k8, v8, out, lse, None)
    dev = _need_gpu(q, k8, v8, workspace, out, lse)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = decode_workspace(q_len, kv_len, hq, hkv, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, q_len), dtype=torch.float32, device=dev)
    st = _on(dev, lib().bca_decode_fp8,
             _ptr(q), _ptr(k8), _ptr(v8), float(k_scale), float(v_scale), _ptr(out), _ptr(lse),
             q_len, kv_len, hq, hkv, d, scale, int(num_splits), _ptr(workspace), ws_bytes,
             _stream(dev))
    _check("bca_decode_fp8", st)
    return out, lse


class DecodeGraph:
    """``steps`` decode calls captured once into a HIP graph (bca_decode_graph_*).

    The graph reads q, k, v and writes out, lse on every launch; write new
    contents into those same tensors between launches.  The tensors are kept
    alive by this object.
    """

    def __init__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, steps: int,
                 scale: Optional[float] = None, num_splits: int = 0,
                 workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None):
        q_len, hq, kv_len, hkv, d = _decode_shapes("DecodeGraph", q, k, v, out, lse,
                                                   torch.bfloat16)
        dev = _need_gpu(q, k, v, workspace, out, lse)
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        need = decode_workspace(q_len, kv_len, hq, hkv, d, num_splits)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self.out = torch.empty_like(q) if out is None else out
        self.lse = torch.empty((hq, q_len), dtype=torch.float32, device=dev) if lse is None else lse
        self._keep = (q, k, v, workspace)
        self._dev = dev
        self._handle = _P()
        st = _on(dev, lib().bca_decode_graph_create,
                 _ptr(q), _ptr(k), _ptr(v), _ptr(self.out), _ptr(self.lse), q_len, kv_len, hq, hkv,
                 d, scale, _dtype_code(q), int(num_splits), _ptr(workspace), ws_bytes, int(steps),
                 ctypes.byref(self._handle))
        _check("bca_decode_graph_create", st)
        self.steps = int(steps)

    def launch(self) -> None:
        """Enqueue one replay (all steps) on torch's current stream."""
        _check("bca_decode_graph_launch",
               _on(self._dev, lib().bca_decode_graph_launch, self._handle,
                   _stream(self._dev)))

    def close(self) -> None:
        """Release the graph after synchronising its device."""
        if self._handle:
            torch.cuda.synchronize(self._dev)
            _on(self._dev, lib().bca_decode_graph_destroy, self._handle)
            self._handle = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DecodeLoop(DecodeGraph):
    """A denoising loop of ``steps`` decode calls captured once
    (bca_decode_loop_create): step i reads q[i] and writes out[i], lse[i];
    every step attends to the first ``kv_len_dev[0]`` rows of the k/v storage,
    read on the GPU when the graph runs, so one graph serves every block.  With
    ``steps_dev`` (int32 on the GPU) only the first ``steps_dev[0]`` steps of a
    replay run; the others leave their outputs untouched."""

    def __init__(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 kv_len_dev: torch.Tensor, scale: Optional[float] = None, num_splits: int = 0,
                 workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, steps_dev: Optional[torch.Tensor] = None):
        if q.dim() != 4:
            raise BcaError("DecodeLoop", 2, "q must be [steps, q_len, hq, d]")
        steps, q_len, hq, d = q.shape
        _decode_shapes("DecodeLoop", q[0], k, v, None, None, torch.bfloat16)
        _expect("DecodeLoop", q, "q", tuple(q.shape), torch.bfloat16)
        _expect("DecodeLoop", out, "out", tuple(q.shape), torch.bfloat16)
        _expect("DecodeLoop", lse, "lse", (steps, hq, q_len), torch.float32)
        for t, name in ((kv_len_dev, "kv_len_dev"), (steps_dev, "steps_dev")):
            if t is not None and (t.dtype != torch.int32 or t.numel() < 1):
                raise BcaError("DecodeLoop", 2, f"{name} must be an int32 tensor")
        dev = _need_gpu(q, k, v, kv_len_dev, steps_dev, workspace, out, lse)
        kv_cap, hkv = k.shape[0], k.shape[1]
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        need = decode_workspace(q_len, kv_cap, hq, hkv, d, num_splits)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self.out = torch.empty_like(q) if out is None else out
        self.lse = (torch.empty((steps, hq, q_len), dtype=torch.float32, device=dev)
                    if lse is None else lse)
        self._keep = (q, k, v, kv_len_dev, steps_dev, workspace)
        self._dev = dev
        self._handle = _P()
        st = _on(dev, lib().bca_decode_loop_create,
                 _ptr(q), _ptr(k), _ptr(v), _ptr(self.out), _ptr(self.lse), _ptr(kv_len_dev),
                 _ptr(steps_dev), q_len, kv_cap, hq, hkv, d, scale, _dtype_code(q), int(num_splits),
                 _ptr(workspace), ws_bytes, int(steps), ctypes.byref(self._handle))
        _check("bca_decode_loop_create", st)
        self.steps = int(steps)


def trajectory_cost(seqlen: int, s_copies: int, block_size: int) -> int:
    """Admitted (query, key) pairs per query head of one trajectory (-1 if invalid)."""
    return int(lib().bca_trajectory_cost(int(seqlen), int(s_copies), int(block_size)))


def pack_balanced(seqlens, s_copies, block_size: int, nbins: int):
    """Compute-balanced assignment of trajectories to ``nbins`` bins (host only).

    Returns numpy arrays (bin_of [ntraj], bin_cost [nbins], order [ntraj],
    bin_start [nbins + 1]); bin b holds order[bin_start[b]:bin_start[b+1]].
    """
    import numpy as np
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    sc = None if s_copies is None else np.ascontiguousarray(np.asarray(s_copies, dtype=np.int32))
    n = int(sl.shape[0])
    if sc is not None and sc.shape[0] != n:
        raise BcaError("bca_pack_balanced", 2, "s_copies must have one entry per trajectory")
    bin_of = np.zeros(n, dtype=np.int32)
    bin_cost = np.zeros(max(int(nbins), 1), dtype=np.int64)
    order = np.zeros(n, dtype=np.int32)
    bin_start = np.zeros(max(int(nbins), 1) + 1, dtype=np.int32)
    vp = lambda a: None if a is None else a.ctypes.data_as(_P)
    st = lib().bca_pack_balanced(vp(sl), vp(sc), n, int(block_size), int(nbins), vp(bin_of),
                                 vp(bin_cost), vp(order), vp(bin_start))
    if st != 0:
        raise BcaError("bca_pack_balanced", st, lib().bca_pack_last_error().decode())
    return bin_of, bin_cost, order, bin_start


def _group_arrays(groups):
    """(group_start [n+1], group_pe, group_copies) int32 host arrays from a
    list, per trajectory, of (pe, copies) groups."""
    import numpy as np
    start = np.zeros(len(groups) + 1, dtype=np.int32)
    start[1:] = np.cumsum([len(g) for g in groups])
    pe = np.ascontiguousarray([int(p) for g in groups for p, _ in g], dtype=np.int32)
    cp = np.ascontiguousarray([int(c) for g in groups for _, c in g], dtype=np.int32)
    return start, pe, cp


def trajectory_cost_groups(seqlen: int, groups, block_size: int) -> int:
    """Admitted pairs per query head of one general-staircase trajectory with
    copy groups [(pe, copies), ...] (-1 if invalid)."""
    _, pe, cp = _group_arrays([groups])
    vp = lambda a: a.ctypes.data_as(_P) if a.size else None
    return int(lib().bca_trajectory_cost_groups(int(seqlen), vp(pe), vp(cp), int(pe.size),
                                                int(block_size)))


def pack_balanced_groups(seqlens, groups, block_size: int, nbins: int):
    """pack_balanced for general-staircase trajectories (copy groups per trajectory)."""
    import numpy as np
    sl = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    n = int(sl.shape[0])
    if len(groups) != n:
        raise BcaError("bca_pack_balanced_groups", 2, "one group list per trajectory")
    start, pe, cp = _group_arrays(groups)
    bin_of = np.zeros(n, dtype=np.int32)
    bin_cost = np.zeros(max(int(nbins), 1), dtype=np.int64)
    order = np.zeros(n, dtype=np.int32)
    bin_start = np.zeros(max(int(nbins), 1) + 1, dtype=np.int32)
    vp = lambda a: a.ctypes.data_as(_P) if a.size else None
    st = lib().bca_pack_balanced_groups(vp(sl), vp(start), vp(pe), vp(cp), n, int(block_size),
                                        int(nbins), vp(bin_of), vp(bin_cost), vp(order),
                                        vp(bin_start))
    if st != 0:
        raise BcaError("bca_pack_balanced_groups", st, lib().bca_pack_last_error().decode())
    return bin_of, bin_cost, order, bin_start
