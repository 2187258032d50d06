"""Plain fp64 CPU oracle for block-causal and staircase attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code with the HIP library.

What it computes follows "On-Policy Residual Learning for Diffusion Language
Models":
  * block-causal attention (thread page, highlight 3): a query in block
    b = floor(i / B) attends bidirectionally to every key of its own block and
    to every key of the earlier blocks;
  * staircase packed replay (paper cards page, Figure 3 caption; thread page,
    Insight 3): each trajectory is a clean prefix of P tokens followed by S
    copies of one B-token block.  Prefix rows are block-causal inside the
    prefix; a row of copy c attends to the whole prefix and to copy c only.
  * the decode step (thread page, Result 4): one block of noisy queries
    attends, unmasked, to the prefix KV cache plus the block's own keys.

Readings taken where the pages are silent (each is restated in the design
notes): block indices are relative to the start of each packed segment and no
query attends across segments; a final partial block (segment length not a
multiple of B, no copies) is bidirectional among its own tokens; the scale is
applied to the scores before the exponential; the log-sum-exp is the natural
logarithm of the sum of exponentials of the scaled scores over the admitted
keys; query head h reads KV head floor(h / (Hq / Hkv)).

Everything here is the plain definition, evaluated densely in float64 on
exactly the input values the GPU sees (bf16 inputs are upcast losslessly): a
masked softmax, its product with V, and the textbook gradients of that
expression.  Rows are processed in chunks only to bound memory.
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 512


def _f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a (CPU) torch tensor of any float dtype."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def segment_prefix_len(seqlen: int, copies: int, block_size: int) -> int:
    """Prefix length P = L - S * B of a segment of L tokens holding S copies."""
    P = seqlen - copies * block_size
    if P < 0:
        raise ValueError(f"segment of {seqlen} tokens cannot hold {copies} copies of {block_size}")
    if copies > 0 and P % block_size != 0:
        raise ValueError("with copies present the prefix must be a whole number of blocks")
    return P


def allowed_matrix(seqlen: int, copies: int, block_size: int) -> np.ndarray:
    """allowed[i, j] (bool, L x L): may query i of the segment attend to key j.

    Prefix rows i < P: j < P and floor(j/B) <= floor(i/B)  (block-causal).
    Copy rows i >= P with c = floor((i - P) / B): j < P, or
    P + c B <= j < P + (c + 1) B  (whole prefix plus its own copy only).
    With no copies (S = 0) this is plain block-causal attention.
    """
    B = block_size
    P = segment_prefix_len(seqlen, copies, B)
    i = np.arange(seqlen)[:, None]
    j = np.arange(seqlen)[None, :]
    prefix_rows = (j < P) & ((j // B) <= (i // B))
    c = (i - P) // B
    copy_rows = (j < P) | ((j >= P + c * B) & (j < P + (c + 1) * B))
    return np.where(i < P, prefix_rows, copy_rows)


def allowed_matrix_groups(seqlen: int, groups, block_size: int) -> np.ndarray:
    """allowed[i, j] for a general trajectory staircase segment.

    ``groups`` lists (pe, copies) in segment order: after the clean prefix of
    P = L - B * (total copies) tokens come the copies of group 0, then of
    group 1, ...; a copy of group g is a noisy state of the block starting at
    clean position pe and sees the clean keys [0, pe) plus, bidirectionally,
    its own B tokens.  Clean rows are block-causal inside the prefix.  Every
    pe must be a multiple of B in [0, P], non-decreasing along the segment.
    """
    B = block_size
    total_copies = sum(int(c) for _, c in groups)
    P = segment_prefix_len(seqlen, total_copies, B)
    prev = 0
    for pe, c in groups:
        if c < 0 or pe % B != 0 or not (0 <= pe <= P) or pe < prev:
            raise ValueError(f"bad copy group (pe={pe}, copies={c}) for P={P}, B={B}")
        prev = pe
    i = np.arange(seqlen)[:, None]
    j = np.arange(seqlen)[None, :]
    allowed = (i < P) & (j < P) & ((j // B) <= (i // B))
    row = P
    for pe, c in groups:
        for _ in range(int(c)):
            own = slice(row, row + B)
            allowed[own, :pe] = True
            allowed[own, own] = True
            row += B
    return allowed


def segment_allowed(seqlen: int, spec, block_size: int) -> np.ndarray:
    """Admitted-key matrix of one segment: ``spec`` is a copy count S (one
    group seeing the whole prefix) or a list of (pe, copies) groups."""
    if isinstance(spec, (list, tuple)):
        return allowed_matrix_groups(seqlen, spec, block_size)
    return allowed_matrix(seqlen, int(spec), block_size)


def _segment_specs(s_copies, nseq: int):
    if s_copies is None:
        return [0] * nseq
    return [x if isinstance(x, (list, tuple)) else int(x) for x in s_copies]


def _kv_head(h: int, hq: int, hkv: int) -> int:
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    return h // (hq // hkv)


def attention_fwd(q, k, v, cu_seqlens, s_copies, block_size: int, scale: float,
                  heads=None, rows=None):
    """Forward pass: O and LSE.

    q: [total, hq, d], k/v: [total, hkv, d]; cu_seqlens int [nseq + 1];
    s_copies int [nseq] (None = all zero).  Returns (O [total, hq, d] float64,
    LSE [hq, total] float64).  ``heads`` restricts the query heads computed and
    ``rows`` (global token indices) the query rows; entries not computed are NaN.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    total, hq, d = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    sc = _segment_specs(s_copies, nseq)
    heads = range(hq) if heads is None else heads
    want = np.ones(total, bool) if rows is None else np.isin(np.arange(total), rows)

    O = np.full((total, hq, d), np.nan)
    LSE = np.full((hq, total), np.nan)
    for s in range(nseq):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        if L == 0:
            continue
        allowed = segment_allowed(L, sc[s], block_size)
        local_rows = np.nonzero(want[a:b])[0]
        for h in heads:
            g = _kv_head(h, hq, hkv)
            K = k[a:b, g, :]
            V = v[a:b, g, :]
            for c0 in range(0, len(local_rows), ROW_CHUNK):
                r = local_rows[c0:c0 + ROW_CHUNK]
                X = scale * (q[a + r, h, :] @ K.T)
                X = np.where(allowed[r], X, -np.inf)
                m = X.max(axis=1, keepdims=True)
                E = np.exp(X - m)
                l = E.sum(axis=1, keepdims=True)
                O[a + r, h, :] = (E / l) @ V
                LSE[h, a + r] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_bwd(q, k, v, do, cu_seqlens, s_copies, block_size: int, scale: float):
    """Forward and backward: returns (O, LSE, dQ, dK, dV), all float64.

    For each segment and query head h with KV head g, with Pm the masked
    softmax of scale * Q_h K_g^T:
      dV_g += Pm^T dO_h;  dP = dO_h V_g^T;  delta = rowsum(dO_h * O_h);
      dS = Pm * (dP - delta);  dQ_h = scale dS K_g;  dK_g += scale dS^T Q_h.
    dK and dV of a KV head sum the contributions of all query heads that read it.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    total, hq, d = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    sc = _segment_specs(s_copies, nseq)

    O = np.zeros((total, hq, d))
    LSE = np.zeros((hq, total))
    dQ = np.zeros((total, hq, d))
    dK = np.zeros((total, hkv, d))
    dV = np.zeros((total, hkv, d))
    for s in range(nseq):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        if L == 0:
            continue
        allowed = segment_allowed(L, sc[s], block_size)
        for h in range(hq):
            g = _kv_head(h, hq, hkv)
            K = k[a:b, g, :]
            V = v[a:b, g, :]
            for r0 in range(0, L, ROW_CHUNK):
                r = np.arange(r0, min(L, r0 + ROW_CHUNK))
                Qh = q[a + r, h, :]
                dOh = do[a + r, h, :]
                X = np.where(allowed[r], scale * (Qh @ K.T), -np.inf)
                m = X.max(axis=1, keepdims=True)
                E = np.exp(X - m)
                l = E.sum(axis=1, keepdims=True)
                Pm = E / l
                Oh = Pm @ V
                O[a + r, h, :] = Oh
                LSE[h, a + r] = (m + np.log(l))[:, 0]
                dV[a:b, g, :] += Pm.T @ dOh
                dP = dOh @ V.T
                delta = np.sum(dOh * Oh, axis=1, keepdims=True)
                dS = Pm * (dP - delta)
                dQ[a + r, h, :] = scale * (dS @ K)
                dK[a:b, g, :] += scale * (dS.T @ Qh)
    return O, LSE, dQ, dK, dV


def decode(q, k, v, scale: float):
    """Decode step: every query of the block attends to every key, unmasked.

    q: [B, hq, d] (the block's queries); k/v: [P + B, hkv, d] (prefix cache
    followed by the block's own keys/values).  Returns (O [B, hq, d],
    LSE [hq, B]), float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Bq, hq, d = q.shape
    hkv = k.shape[1]
    O = np.zeros((Bq, hq, d))
    LSE = np.zeros((hq, Bq))
    for h in range(hq):
        g = _kv_head(h, hq, hkv)
        X = scale * (q[:, h, :] @ k[:, g, :].T)
        m = X.max(axis=1, keepdims=True)
        E = np.exp(X - m)
        l = E.sum(axis=1, keepdims=True)
        O[:, h, :] = (E / l) @ v[:, g, :]
        LSE[h, :] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_dq_rows(q, k, v, do, cu_seqlens, s_copies, block_size: int, scale: float,
                      rows, heads=None):
    """dQ for selected query rows only (each row's gradient needs only that row).

    Returns dQ [total, hq, d] float64 with NaN outside (rows x heads).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    total, hq, d = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    sc = _segment_specs(s_copies, nseq)
    heads = range(hq) if heads is None else heads
    rows = np.asarray(rows, dtype=np.int64)
    dQ = np.full((total, hq, d), np.nan)
    for s in range(nseq):
        a, b = int(cu[s]), int(cu[s + 1])
        r = rows[(rows >= a) & (rows < b)] - a
        if len(r) == 0:
            continue
        allowed = segment_allowed(b - a, sc[s], block_size)[r]
        for h in heads:
            g = _kv_head(h, hq, hkv)
            K = k[a:b, g, :]
            V = v[a:b, g, :]
            X = np.where(allowed, scale * (q[a + r, h, :] @ K.T), -np.inf)
            m = X.max(axis=1, keepdims=True)
            E = np.exp(X - m)
            Pm = E / E.sum(axis=1, keepdims=True)
            Oh = Pm @ V
            dOh = do[a + r, h, :]
            dS = Pm * (dOh @ V.T - np.sum(dOh * Oh, axis=1, keepdims=True))
            dQ[a + r, h, :] = scale * (dS @ K)
    return dQ
