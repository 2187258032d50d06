"""Seeded synthetic inputs for block-causal / staircase attention.

This module draws random tensors and segment lengths and nothing else: it
holds none of the attention arithmetic, so both the fp64 oracle (through the
tests) and the HIP path consume the very same inputs from it.

The workloads stand in for the benchmark-driven serving and training runs of
"On-Policy Residual Learning for Diffusion Language Models" (paper cards page,
Tables 5, 9 and 14): 32 query heads sharing 8 KV heads of width 128 (Table 9's
QKV projection 2560 -> 6144 = 32*128 + 2*8*128), block size 32 (thread page,
Result 2) and irregular trajectories (thread page, Insight 3).  No dataset or
trained weight is involved; every value is N(0, 1).

Draw order per workload (one ``numpy.random.default_rng(seed)`` each): segment
lengths (all prefixes, then all copy counts), then Q, K, V and, for the
backward, dO.  Each tensor is drawn as float32 standard normals and, for bf16
workloads, rounded to bf16 with round-to-nearest-even (torch CPU cast).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass
class Workload:
    """One attention problem, packed varlen, host-resident.

    Tensors are row-major: q and o are [total, hq, d]; k and v are
    [total, hkv, d] (decode: [kv_len, hkv, d]); cu_seqlens is int32
    [nseq + 1]; s_copies is int32 [nseq] (all zero for plain block-causal).
    """

    name: str
    kind: str                 # "fwd", "staircase_fwd", "staircase_bwd", "decode", "staircase_groups"
    dtype: str                # "f32" or "bf16"
    hq: int
    hkv: int
    d: int
    block_size: int
    scale: float
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens: np.ndarray
    s_copies: np.ndarray
    do: Optional[torch.Tensor] = None
    prefix_lens: Optional[np.ndarray] = None
    seed: int = 0
    # general staircase: per segment a list of (prefix end, copies) groups
    groups: Optional[list] = None

    @property
    def total(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def nseq(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def max_seqlen(self) -> int:
        return int(np.max(np.diff(self.cu_seqlens))) if self.nseq else 0

    def group_table(self):
        """(group_start [nseq+1], group_pe [G], group_copies [G]) int32 arrays."""
        if self.groups is None:
            raise ValueError("not a general staircase workload")
        start = np.zeros(self.nseq + 1, dtype=np.int32)
        start[1:] = np.cumsum([len(g) for g in self.groups])
        pe = np.array([p for g in self.groups for p, _ in g], dtype=np.int32)
        cp = np.array([c for g in self.groups for _, c in g], dtype=np.int32)
        return start, pe, cp

    def describe(self) -> dict:
        return {
            "workload": self.name, "kind": self.kind, "dtype": self.dtype,
            "hq": self.hq, "hkv": self.hkv, "d": self.d,
            "block_size": self.block_size, "seed": self.seed,
            "total": self.total, "nseq": self.nseq,
            "seqlens": np.diff(self.cu_seqlens).tolist(),
            "s_copies": self.s_copies.tolist(),
        }


def _draw(rng: np.random.Generator, shape, dtype: str) -> torch.Tensor:
    x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def packed(name: str, kind: str, seed: int, seqlens, s_copies, hq: int, hkv: int,
           d: int, block_size: int, dtype: str, with_do: bool = False,
           scale: Optional[float] = None, rng: Optional[np.random.Generator] = None,
           prefix_lens=None) -> Workload:
    """Packed varlen problem with explicit segment lengths (tokens) and copies."""
    if rng is None:
        rng = np.random.default_rng(seed)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    s_copies = np.asarray(s_copies, dtype=np.int32)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    total = int(cu[-1])
    q = _draw(rng, (total, hq, d), dtype)
    k = _draw(rng, (total, hkv, d), dtype)
    v = _draw(rng, (total, hkv, d), dtype)
    do = _draw(rng, (total, hq, d), dtype) if with_do else None
    return Workload(name=name, kind=kind, dtype=dtype, hq=hq, hkv=hkv, d=d,
                    block_size=block_size,
                    scale=(1.0 / math.sqrt(d)) if scale is None else scale,
                    q=q, k=k, v=v, do=do, cu_seqlens=cu, s_copies=s_copies,
                    prefix_lens=None if prefix_lens is None else np.asarray(prefix_lens),
                    seed=seed)


def staircase_lengths(rng: np.random.Generator, ntraj: int, block_size: int,
                      prefix_blocks_lo: int, prefix_blocks_hi: int,
                      copies_lo: int, copies_hi: int):
    """Trajectory shapes: prefix = block_size * U{lo..hi} tokens, S = U{lo..hi}.

    All prefixes are drawn first, then all copy counts (both bounds inclusive).
    """
    prefix = block_size * rng.integers(prefix_blocks_lo, prefix_blocks_hi + 1, size=ntraj)
    copies = rng.integers(copies_lo, copies_hi + 1, size=ntraj)
    seqlens = prefix + copies * block_size
    return prefix.astype(np.int64), copies.astype(np.int32), seqlens.astype(np.int64)


# ---------------------------------------------------------------------------
# The five named workloads.

def blockcausal_fp32_small() -> Workload:
    """One sequence of 256 tokens, 1 head, d = 64, block 32, fp32, seed 0."""
    return packed("blockcausal_fp32_L256_d64", "fwd", 0, [256], [0], 1, 1, 64, 32, "f32")


def prefill_bf16_4k() -> Workload:
    """Block-causal prefill: 1 x 4096 tokens, 32/8 heads, d = 128, block 32, bf16, seed 1."""
    return packed("prefill_bf16_L4096_gqa32x8_d128_B32", "fwd", 1, [4096], [0], 32, 8, 128,
                  32, "bf16")


def decode_step(prefix_len: int, block_size: int = 32, hq: int = 32, hkv: int = 8,
                d: int = 128, seed: int = 2) -> Workload:
    """One noisy block of ``block_size`` queries against prefix + own K/V (fresh rng per P).

    q is [block_size, hq, d]; k and v are [prefix_len + block_size, hkv, d] with the
    block's own keys and values in the last ``block_size`` rows.
    """
    rng = np.random.default_rng(seed)
    kv_len = prefix_len + block_size
    q = _draw(rng, (block_size, hq, d), "bf16")
    k = _draw(rng, (kv_len, hkv, d), "bf16")
    v = _draw(rng, (kv_len, hkv, d), "bf16")
    cu = np.array([0, block_size], dtype=np.int32)
    return Workload(name=f"decode_bf16_P{prefix_len}_B{block_size}_gqa{hq}x{hkv}_d{d}",
                    kind="decode", dtype="bf16", hq=hq, hkv=hkv, d=d,
                    block_size=block_size, scale=1.0 / math.sqrt(d), q=q, k=k, v=v,
                    cu_seqlens=cu, s_copies=np.zeros(1, np.int32),
                    prefix_lens=np.array([prefix_len]), seed=seed)


def decode_step_fp8(prefix_len: int, block_size: int = 32, hq: int = 32, hkv: int = 8,
                    d: int = 128, seed: int = 7):
    """Decode step against an FP8 E4M3 cache: returns (workload, k8, v8, k_scale, v_scale).

    K and V are drawn as for decode_step, then stored as E4M3 bytes of
    K / k_scale and V / v_scale with per-tensor scales max|x| / 448 (the
    largest E4M3 value), rounded to nearest even by torch's CPU cast; the
    workload's k and v hold the decoded values k_scale * e4m3 (float32).
    """
    w = decode_step(prefix_len, block_size, hq, hkv, d, seed)
    rng = np.random.default_rng(seed + 1000)
    kv_len = prefix_len + block_size
    k = torch.from_numpy(rng.standard_normal((kv_len, hkv, d), dtype=np.float32))
    v = torch.from_numpy(rng.standard_normal((kv_len, hkv, d), dtype=np.float32))
    k_scale = float(k.abs().max()) / 448.0
    v_scale = float(v.abs().max()) / 448.0
    k8 = (k / k_scale).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (v / v_scale).to(torch.float8_e4m3fn).view(torch.uint8)
    w.k = k8.view(torch.float8_e4m3fn).float() * k_scale
    w.v = v8.view(torch.float8_e4m3fn).float() * v_scale
    w.name = f"decode_fp8_P{prefix_len}_B{block_size}_gqa{hq}x{hkv}_d{d}"
    return w, k8, v8, k_scale, v_scale


def staircase_fwd_8traj() -> Workload:
    """8 trajectories, prefix 32*U{16..128}, S = U{4..24} copies of a 32-token block, seed 3."""
    rng = np.random.default_rng(3)
    prefix, copies, seqlens = staircase_lengths(rng, 8, 32, 16, 128, 4, 24)
    return packed("staircase_fwd_bf16_8traj_B32", "staircase_fwd", 3, seqlens, copies,
                  32, 8, 128, 32, "bf16", rng=rng, prefix_lens=prefix)


def staircase_bwd_16traj() -> Workload:
    """16 trajectories, prefix 64*U{16..128}, S = U{4..24} copies of a 64-token block,
    dO drawn after V, seed 4."""
    rng = np.random.default_rng(4)
    prefix, copies, seqlens = staircase_lengths(rng, 16, 64, 16, 128, 4, 24)
    return packed("staircase_fwdbwd_bf16_16traj_B64", "staircase_bwd", 4, seqlens, copies,
                  32, 8, 128, 64, "bf16", with_do=True, rng=rng, prefix_lens=prefix)


def general_staircase(name: str, seed: int, ntraj: int, block_size: int, blocks_lo: int,
                      blocks_hi: int, copies_lo: int, copies_hi: int, hq: int, hkv: int, d: int,
                      dtype: str, with_do: bool = False) -> Workload:
    """Trajectories replayed with a copy group per block.

    Each trajectory has n = U{blocks_lo..blocks_hi} clean blocks (P = n B
    tokens); block b gets U{copies_lo..copies_hi} copies, each seeing the
    clean keys before block b ([0, b B)) and itself.  Draw order: all block
    counts, then the copy counts trajectory by trajectory, block by block,
    then Q, K, V (and dO).
    """
    rng = np.random.default_rng(seed)
    nblocks = rng.integers(blocks_lo, blocks_hi + 1, size=ntraj)
    groups, seqlens, copies = [], [], []
    for n in nblocks.tolist():
        cps = rng.integers(copies_lo, copies_hi + 1, size=n).tolist()
        groups.append([(b * block_size, int(c)) for b, c in enumerate(cps)])
        copies.append(int(sum(cps)))
        seqlens.append(n * block_size + int(sum(cps)) * block_size)
    w = packed(name, "staircase_groups", seed, seqlens, copies, hq, hkv, d, block_size, dtype,
               with_do=with_do, rng=rng, prefix_lens=nblocks * block_size)
    w.groups = groups
    return w


def staircase_groups_8traj() -> Workload:
    """8 trajectories, 8-32 clean blocks of 32 tokens, 1-4 copies per block, dO, seed 6."""
    return general_staircase("staircase_groups_bf16_8traj_B32", 6, 8, 32, 8, 32, 1, 4, 32, 8,
                             128, "bf16", with_do=True)


def useful_pairs(seqlens, s_copies, block_size: int) -> int:
    """Number of (query, key) pairs the attention admits, per query head.

    Counted in closed form per segment: the prefix of n = P / B whole blocks
    (plus a final partial block of r tokens) admits B^2 n(n+1)/2 + r (nB + r)
    pairs, and each of the S copies admits B (P + B).  This is a cost model for
    measurement (useful FLOPs), not part of the attention itself.
    """
    total = 0
    for L, S in zip(np.asarray(seqlens).tolist(), np.asarray(s_copies).tolist()):
        B = block_size
        P = L - S * B
        n, r = divmod(P, B)
        total += B * B * n * (n + 1) // 2 + r * (n * B + r)
        total += S * B * (P + B)
    return int(total)


def useful_pairs_groups(seqlens, groups, block_size: int) -> int:
    """Admitted (query, key) pairs per query head of general staircase
    segments, in closed form: the clean prefix of n whole blocks (plus r
    tokens) as in useful_pairs, and each copy of a group with prefix end pe
    admits B (pe + B) pairs.  A cost model for measurement only."""
    total = 0
    B = block_size
    for L, g in zip(np.asarray(seqlens).tolist(), groups):
        S = sum(c for _, c in g)
        P = L - S * B
        n, r = divmod(P, B)
        total += B * B * n * (n + 1) // 2 + r * (n * B + r)
        total += sum(c * B * (pe + B) for pe, c in g)
    return int(total)
