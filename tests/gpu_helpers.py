"""Shared plumbing of the GPU parity tests: moving workloads to the device,
calling the binding, and comparing with the oracle on chosen rows."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from block_diffusion_lm_causal_amd import bca
from block_diffusion_lm_causal_amd.workloads import Workload

TOL_BF16 = 1e-2   # max-abs on O and LSE for bf16 inputs
TOL_F32 = 1e-5    # max-abs on O and LSE for the float32 path
TOL_GRAD = 1e-2   # max|err| <= TOL_GRAD * max|ref|, per gradient tensor


def gpu_available() -> bool:
    return torch.cuda.is_available()


def device_inputs(w: Workload):
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev).contiguous() for t in (w.q, w.k, w.v))
    cu = torch.from_numpy(np.asarray(w.cu_seqlens, np.int32)).to(dev)
    sc = torch.from_numpy(np.asarray(w.s_copies, np.int32)).to(dev)
    do = None if w.do is None else w.do.to(dev).contiguous()
    return q, k, v, cu, sc, do


def run_fwd(w: Workload, staircase: bool = True):
    q, k, v, cu, sc, _ = device_inputs(w)
    if staircase:
        o, lse = bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen)
    else:
        o, lse = bca.fwd(q, k, v, cu, w.block_size, w.scale, w.max_seqlen)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def segment_spec(w: Workload, s: int):
    """The oracle's copy description of segment s: its copy groups, or S."""
    return w.groups[s] if w.groups is not None else int(w.s_copies[s])


def group_tensors(w: Workload):
    dev = torch.device("cuda", 0)
    return tuple(torch.from_numpy(x).to(dev) for x in w.group_table())


def run_groups_fwd(w: Workload):
    q, k, v, cu, _, _ = device_inputs(w)
    gs, gp, gc = group_tensors(w)
    o, lse = bca.staircase_groups_fwd(q, k, v, cu, gs, gp, gc, w.block_size, w.scale,
                                      w.max_seqlen)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_rows(w: Workload, rows, heads=None):
    """Oracle O/LSE on selected global rows, one segment at a time."""
    rows = np.unique(np.asarray(rows, np.int64))
    O = np.full((w.total, w.hq, w.d), np.nan)
    LSE = np.full((w.hq, w.total), np.nan)
    cu = np.asarray(w.cu_seqlens, np.int64)
    for s in range(w.nseq):
        a, b = int(cu[s]), int(cu[s + 1])
        r = rows[(rows >= a) & (rows < b)]
        if len(r) == 0:
            continue
        o, lse = oracle.attention_fwd(w.q[a:b], w.k[a:b], w.v[a:b], [0, b - a],
                                      [segment_spec(w, s)], w.block_size, w.scale,
                                      heads=heads, rows=r - a)
        O[a:b][r - a] = o[r - a]
        LSE[:, a:b][:, r - a] = lse[:, r - a]
    return O, LSE


def sample_rows(w: Workload, rng: np.random.Generator, per_segment: int = 6):
    """Rows that exercise every tile kind: segment ends, block and tile edges,
    the prefix/copy boundary, plus random ones."""
    rows = []
    cu = np.asarray(w.cu_seqlens, np.int64)
    B = w.block_size
    for s in range(w.nseq):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        if L == 0:
            continue
        P = L - int(w.s_copies[s]) * B
        cand = [0, L - 1, min(L - 1, B - 1), min(L - 1, B), P - 1, P, P + B - 1, P + B,
                min(L - 1, 31), min(L - 1, 32), min(L - 1, 127), min(L - 1, 128)]
        if w.groups is not None:  # first and last row of every copy group
            row = P
            for _, c in w.groups[s]:
                if c:
                    cand += [row, row + c * B - 1]
                row += c * B
        cand += rng.integers(0, L, size=per_segment).tolist()
        rows += [a + c for c in cand if 0 <= c < L]
    return np.unique(rows)


def max_abs(a, b, mask=None):
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    if mask is not None:
        d = d[mask]
    return float(np.max(d)) if d.size else 0.0
