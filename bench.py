#!/usr/bin/env python3
"""Benchmark of block-causal / staircase attention on one MI355X.

Headline (``value``): useful TFLOP/s of one training step of the staircase
packed replay -- forward and backward over 16 packed trajectories (prefix of
64 * U{16..128} tokens, then U{4..24} copies of one 64-token block), 32 query
heads sharing 8 KV heads, head_dim 128, bf16 -- counting 4 * d FLOPs per
admitted query-key pair per query head for the forward and 10 * d for the
backward (masked pairs and padded tiles are not counted).  One step is the
forward call plus the backward call (the row-term, dK/dV and dQ kernels),
inputs resident in HBM.

``roofline`` is that of the step's dominant kernel, the dK/dV kernel of the
backward: its algorithmic work is the four products S = Q K^T, dP = dO V^T,
dV += P^T dO and dK += dS^T Q, 8 * d FLOPs per admitted pair per query head,
over its mean duration from HIP events on the launch stream; ``traffic`` its
HBM bytes per launch from the committed rocprofv3 counter summary (only while
the kernel's sources are those the counters were taken with).

``measured_peaks``: the machine's own MFMA rate and clock under MFMA load, its
streaming-read bandwidth (1 GiB) and a cold 34 MB read, and the event-timed
cost of an empty kernel (the floor under every single-call figure).

``paths``: the 4096-token block-causal prefill (with its own roofline), the
decode step against a prefix of 1024 or 8192 keys (bf16 and FP8 caches: HBM
GB/s of the algorithmic bytes -- K and V read once per KV head, Q read, O and
LSE written -- per flushed call, warm, per step of a captured 32-step loop,
and per step of a captured loop that reads 512 MB between steps as the
model's weight stream does), the 8-trajectory staircase forward, the copy-group
staircase forward and backward, and the packing routine.

``cpu_baseline``: the fp64 CPU oracle on a bounded sample of the headline
workload, plus bounded samples of every other workload (``per_config``), on
the host's BLAS threads.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-cpu]
       [--paths prefill,decode,staircase,groups,packing,peaks,decode_calls] [--skip-headline]
       [--copy-calibration]
Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU (the 2.5 PFLOP/s figure)
PEAK_HBM_GBS = 8000.0      # HBM3E, 8 TB/s
PROFILES = os.path.join(ROOT, "profiles")
PKG = os.path.join(ROOT, "block_diffusion_lm_causal_amd")
CSRC = os.path.join(PKG, "csrc")
HEADLINE = "staircase_fwdbwd_bf16_16traj_B64"
ALL_PATHS = "prefill,decode,staircase,groups,packing,peaks"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# Sources each measured kernel is built from: stored HBM-traffic counters are
# used only while these hash to the digest recorded with the counters.
FWD_SOURCES = ("attn_fwd_bf16.hip", "attn_common.hpp", "bca_device.hpp", "bca_kernels.hpp")
BWD_SOURCES = ("attn_bwd_bf16.hip", "bca_device.hpp", "bca_kernels.hpp")
DECODE_SOURCES = ("attn_decode_bf16.hip", "attn_common.hpp", "bca_device.hpp", "bca_kernels.hpp")
KERNEL_SOURCES = {
    "fwd_bf16_prefill_L4096": FWD_SOURCES,
    "bwd_dkdv_16traj_B64": BWD_SOURCES,
    "decode_bf16_P1024": DECODE_SOURCES,
    "decode_bf16_P8192": DECODE_SOURCES,
}


def source_digest(files=FWD_SOURCES) -> str:
    """Hash of a kernel's sources."""
    h = hashlib.sha256()
    for name in sorted(files):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_tag: str, files=None):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken with the current kernel sources (else None)."""
    files = files or KERNEL_SOURCES.get(kernel_tag, FWD_SOURCES)
    path = os.path.join(PROFILES, f"{kernel_tag}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != source_digest(files):
        return None
    return float(m_val.group(1))


def warm_up(fn, warmup: int) -> None:
    """W calls, continued until about a second of work has run so that the GPU
    clocks have settled before a timed region."""
    import torch
    t_warm = time.perf_counter()
    done = 0
    while done < warmup or (time.perf_counter() - t_warm < 1.0 and done < 20 * max(warmup, 1)):
        fn()
        done += 1
        if done % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed_calls(fn, steps: int, warmup: int, flush=None):
    """Run fn() warmup + steps times; returns (per-call event ms list, wall ms of the
    timed region).  With flush, the cache flush runs before every timed call,
    outside its events, and the wall figure is not meaningful."""
    import torch
    warm_up(fn, warmup)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    return [s.elapsed_time(e) for s, e in zip(starts, ends)], wall_ms


class Probe:
    """libbca_probe.so: the machine microbenchmarks (read, MFMA, empty kernel)."""

    def __init__(self):
        import torch
        path = os.path.join(PKG, "libbca_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing; build with `python -m "
                               "block_diffusion_lm_causal_amd.build`")
        self.L = ctypes.CDLL(path)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        self.L.bca_probe_read.argtypes = [P, S, I, P, P]
        self.L.bca_probe_mfma.argtypes = [I, I, P, P, P]
        self.L.bca_probe_empty.argtypes = [P]
        self.L.bca_probe_mfma_lds.argtypes = [I, I, I, P, P, P]
        self.L.bca_probe_valu.argtypes = [I, I, I, P, P, P]
        self.sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")

    @staticmethod
    def stream():
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def read(self, buf, nbytes: int, wgs: int = 256) -> None:
        rc = self.L.bca_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes // 16 * 16, wgs,
                                   ctypes.c_void_p(self.sink.data_ptr()), self.stream())
        if rc != 0:
            raise RuntimeError(f"probe read launch failed ({rc})")

    def empty(self) -> None:
        if self.L.bca_probe_empty(self.stream()) != 0:
            raise RuntimeError("probe launch failed")


def make_flush(dev, probe: Probe):
    """Evict L2 and the Infinity Cache before a timed call by READING 512 MB
    (a decode loop streams the model's weights between steps).  A write-based
    flush would leave dirty lines whose write-back competes with the call."""
    import torch
    buf = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    return buf, (lambda: probe.read(buf, buf.numel() * 4))


def bench_headline(steps: int, warmup: int):
    """Forward + backward of the 16-trajectory staircase, each kernel bracketed
    by events on the launch stream; wall time over the steps for ``value``."""
    import numpy as np
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    w = workloads.staircase_bwd_16traj()
    dev = torch.device("cuda", 0)
    q, k, v, do = (t.to(dev) for t in (w.q, w.k, w.v, w.do))
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    sc = torch.from_numpy(w.s_copies).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.total), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(bca.staircase_bwd_workspace(w.total, w.hq, w.hkv, w.d), dtype=torch.uint8,
                     device=dev)
    pairs = workloads.useful_pairs(np.diff(w.cu_seqlens), w.s_copies, w.block_size)
    B, S, ms = w.block_size, w.scale, w.max_seqlen

    def fwd():
        bca.staircase_fwd(q, k, v, cu, sc, B, S, ms, out=o, lse=lse)

    def bwd(stage=0):
        bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, B, S, ms, workspace=ws, dq=dq, dk=dk,
                          dv=dv, stage=stage)

    # The step as a caller runs it: the forward call, then the whole backward
    # call (stage 0: its three kernels back to back).
    def step():
        fwd()
        bwd()

    warm_up(step, warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record()
        fwd()
        ev[i][1].record()
        bwd()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    step_ms = {"fwd": statistics.mean(e[0].elapsed_time(e[1]) for e in ev),
               "bwd": statistics.mean(e[1].elapsed_time(e[2]) for e in ev)}
    # Each backward kernel on its own (stages 1-3), for the per-kernel figures
    # and the dK/dV roofline.
    calls = [fwd] + [lambda st=stage: bwd(st) for stage in (1, 2, 3)]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        for j, c in enumerate(calls):
            c()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    names = ["fwd_pp_kernel<128>", "bwd_delta_kernel", "bwd_dkdv_pp_kernel<128>",
             "bwd_dq_kernel<128>"]
    kms = {n: statistics.mean(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps))
           for j, n in enumerate(names)}
    return w, pairs, kms, wall_ms, step_ms


def bench_prefill(steps: int, warmup: int):
    import numpy as np
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    w = workloads.prefill_bf16_4k()
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.total), dtype=torch.float32, device=dev)
    pairs = workloads.useful_pairs(np.diff(w.cu_seqlens), w.s_copies, w.block_size)
    flops = 4.0 * w.d * pairs * w.hq

    def step():
        bca.fwd(q, k, v, cu, w.block_size, w.scale, w.max_seqlen, out=o, lse=lse)

    per_call, wall = timed_calls(step, steps, warmup)
    kernel_ms = statistics.mean(per_call)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    return {"workload": w.name, "useful_pairs_per_head": pairs, "flops": flops,
            "ms_per_call_wall": round(wall / steps, 5), "kernel_ms_mean_events": round(kernel_ms, 5),
            "TFLOPs": round(achieved, 1),
            "roofline": {"bound": "mfma", "kernel": "fwd_pp_kernel<128>",
                         "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                         "traffic": stored_traffic("fwd_bf16_prefill_L4096")}}


def decode_loop_graphs(step, flush_read, steps: int):
    """Per-step ms of a captured loop of `steps` decode calls, and of the same
    loop with the 512 MB read before every call minus a loop of reads alone.
    Returns (warm_ms, cold_ms, read_ms)."""
    import torch

    def capture(body):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            body()  # one eager pass on the capture stream before capturing
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            body()
        torch.cuda.synchronize()
        return g

    def loop(with_decode, with_read):
        def body():
            for _ in range(steps):
                if with_read:
                    flush_read()
                if with_decode:
                    step()
        return body

    out = []
    for wd, wr in ((True, False), (True, True), (False, True)):
        g = capture(loop(wd, wr))
        per, _ = timed_calls(g.replay, 10, 2)
        out.append(statistics.median(per) / steps)
        del g
    warm, both, reads = out
    return warm, both - reads, reads


def bench_decode(prefix: int, probe: Probe, flush, flush_read, calls: int = 32, fp8: bool = False):
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    dev = torch.device("cuda", 0)
    if fp8:
        w, k8, v8, ks, vs = workloads.decode_step_fp8(prefix)
        q, k, v = w.q.to(dev), k8.to(dev), v8.to(dev)
        elem = 1
    else:
        w = workloads.decode_step(prefix)
        q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
        elem = 2
    kv_len = prefix + w.block_size
    ws = torch.empty(max(bca.decode_workspace(w.block_size, kv_len, w.hq, w.hkv, w.d), 16),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.block_size), dtype=torch.float32, device=dev)
    algo_bytes = (2 * kv_len * w.hkv * w.d * elem + 2 * w.block_size * w.hq * w.d * 2
                  + w.hq * w.block_size * 4)

    if fp8:
        def step():
            bca.decode_fp8(q, k, v, ks, vs, w.scale, workspace=ws, out=o, lse=lse)
    else:
        def step():
            bca.decode(q, k, v, w.scale, workspace=ws, out=o, lse=lse)

    cold, _ = timed_calls(step, calls, 3, flush=flush)
    warm, _ = timed_calls(step, calls, 3)
    cold_us = statistics.median(cold) * 1e3
    warm_us = statistics.median(warm) * 1e3
    gwarm, gcold, gread = decode_loop_graphs(step, flush_read, calls)
    gb = lambda us: round(algo_bytes / us / 1e3, 1)
    res = {
        "workload": w.name, "bytes_per_call": algo_bytes, "calls": calls,
        "us_per_call_flushed_median": round(cold_us, 3),
        "GBps_flushed": gb(cold_us),
        "frac_hbm_flushed": round(algo_bytes / cold_us / 1e3 / PEAK_HBM_GBS, 4),
        "us_per_call_warm_median": round(warm_us, 3),
        "us_per_step_graph_replay_warm": round(gwarm * 1e3, 3),
        "GBps_graph_replay_warm": gb(gwarm * 1e3),
        "us_per_step_graph_replay_512MB_read_between": round(gcold * 1e3, 3),
        "GBps_graph_replay_512MB_read_between": gb(gcold * 1e3),
        "frac_hbm_graph_replay_512MB_read_between": round(
            algo_bytes / (gcold * 1e3) / 1e3 / PEAK_HBM_GBS, 4),
        "us_512MB_read_alone_per_step": round(gread * 1e3, 2),
    }
    if not fp8:
        # the captured loop with a device-resident cache length (one graph for
        # every block of a generation), 32 steps per replay, caches warm
        qs = q.unsqueeze(0).repeat(calls, 1, 1, 1).contiguous()
        kv_len_dev = torch.full((1,), kv_len, dtype=torch.int32, device=dev)
        loop = bca.DecodeLoop(qs, k, v, kv_len_dev, w.scale)
        try:
            per, _ = timed_calls(loop.launch, 10, 2)
        finally:
            loop.close()
        res["us_per_step_device_len_loop_warm"] = round(statistics.median(per) * 1e3 / calls, 3)
        res["roofline_graph_cold"] = {
            "bound": "hbm", "achieved": gb(gcold * 1e3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(algo_bytes / (gcold * 1e3) / 1e3 / PEAK_HBM_GBS, 4),
            "traffic": stored_traffic(f"decode_bf16_P{prefix}")}
    return res


def bench_decode_calls(prefix: int, flush, calls: int = 16):
    """Only the flushed decode calls (bf16 cache), for counter runs."""
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    dev = torch.device("cuda", 0)
    w = workloads.decode_step(prefix)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    kv_len = prefix + w.block_size
    ws = torch.empty(max(bca.decode_workspace(w.block_size, kv_len, w.hq, w.hkv, w.d), 16),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.block_size), dtype=torch.float32, device=dev)
    cold, _ = timed_calls(lambda: bca.decode(q, k, v, w.scale, workspace=ws, out=o, lse=lse),
                          calls, 2, flush=flush)
    return {"workload": w.name, "calls": calls,
            "us_per_call_flushed_median": round(statistics.median(cold) * 1e3, 3)}


def bench_decode_splits(flush, calls: int = 32):
    """Flushed median per decode call for a range of split counts (0 = the
    library's own plan), bf16 and FP8 caches, P = 1024 and 8192."""
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    dev = torch.device("cuda", 0)
    res = {}
    for prefix in (1024, 8192):
        tiles = (prefix + 32 + 63) // 64
        counts = [0] + [n for n in (1, 2, 3, 4, 6, 8, 9, 13, 17, 22, 26, 32) if n <= tiles]
        for fp8 in (False, True):
            if fp8:
                w, k8, v8, ks, vs = workloads.decode_step_fp8(prefix)
                q, k, v = w.q.to(dev), k8.to(dev), v8.to(dev)
            else:
                w = workloads.decode_step(prefix)
                q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
            kv_len = prefix + w.block_size
            o = torch.empty_like(q)
            lse = torch.empty((w.hq, w.block_size), dtype=torch.float32, device=dev)
            per = {}
            for ns in counts:
                ws = torch.empty(max(bca.decode_workspace(w.block_size, kv_len, w.hq, w.hkv, w.d,
                                                          ns), 16), dtype=torch.uint8, device=dev)
                if fp8:
                    def step():
                        bca.decode_fp8(q, k, v, ks, vs, w.scale, num_splits=ns, workspace=ws,
                                       out=o, lse=lse)
                else:
                    def step():
                        bca.decode(q, k, v, w.scale, num_splits=ns, workspace=ws, out=o, lse=lse)
                cold, _ = timed_calls(step, calls, 3, flush=flush)
                per["plan" if ns == 0 else str(ns)] = round(statistics.median(cold) * 1e3, 3)
            res[w.name] = {"us_per_call_flushed_median_by_splits": per}
    return res


def bench_staircase8(steps: int, warmup: int):
    import numpy as np
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    w = workloads.staircase_fwd_8traj()
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    sc = torch.from_numpy(w.s_copies).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.total), dtype=torch.float32, device=dev)
    pairs = workloads.useful_pairs(np.diff(w.cu_seqlens), w.s_copies, w.block_size)
    fwd_flops = 4.0 * w.d * pairs * w.hq

    def fwd():
        bca.staircase_fwd(q, k, v, cu, sc, w.block_size, w.scale, w.max_seqlen, out=o, lse=lse)

    per_call, _ = timed_calls(fwd, steps, warmup)
    fwd_ms = statistics.median(per_call)
    return {"workload": w.name, "total_tokens": w.total, "useful_pairs_per_head": pairs,
            "fwd_ms_median": round(fwd_ms, 4),
            "fwd_TFLOPs": round(fwd_flops / fwd_ms / 1e9, 1),
            "fwd_frac_mfma": round(fwd_flops / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}


def bench_groups(steps: int, warmup: int):
    """General trajectory staircase (a copy group per block), forward and backward."""
    import numpy as np
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    w = workloads.staircase_groups_8traj()
    dev = torch.device("cuda", 0)
    q, k, v, do = (t.to(dev) for t in (w.q, w.k, w.v, w.do))
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    gs, gp, gc = (torch.from_numpy(x).to(dev) for x in w.group_table())
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.total), dtype=torch.float32, device=dev)
    pairs = workloads.useful_pairs_groups(np.diff(w.cu_seqlens), w.groups, w.block_size)

    def fwd():
        bca.staircase_groups_fwd(q, k, v, cu, gs, gp, gc, w.block_size, w.scale, w.max_seqlen,
                                 out=o, lse=lse)

    per_call, _ = timed_calls(fwd, steps, warmup)
    fwd_ms = statistics.median(per_call)
    ws = torch.empty(bca.staircase_bwd_workspace(w.total, w.hq, w.hkv, w.d), dtype=torch.uint8,
                     device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fwd()

    def bwd():
        bca.staircase_groups_bwd(q, k, v, o, lse, do, cu, gs, gp, gc, w.block_size, w.scale,
                                 w.max_seqlen, workspace=ws, dq=dq, dk=dk, dv=dv)

    per_call, _ = timed_calls(bwd, steps, warmup)
    bwd_ms = statistics.median(per_call)
    fwd_flops, bwd_flops = 4.0 * w.d * pairs * w.hq, 10.0 * w.d * pairs * w.hq
    return {"workload": w.name, "total_tokens": w.total, "groups": int(gp.numel()),
            "useful_pairs_per_head": pairs,
            "fwd_ms_median": round(fwd_ms, 4),
            "fwd_TFLOPs": round(fwd_flops / fwd_ms / 1e9, 1),
            "fwd_frac_mfma": round(fwd_flops / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "bwd_ms_median": round(bwd_ms, 4),
            "bwd_TFLOPs_10d": round(bwd_flops / bwd_ms / 1e9, 1),
            "bwd_frac_mfma_10d": round(bwd_flops / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}


def bench_packing():
    """Compute-balanced packing (host): balance of the 16-trajectory workload
    over 8 bins, and the time to pack 10,000 random trajectories."""
    import numpy as np
    from block_diffusion_lm_causal_amd import bca, workloads
    w = workloads.staircase_bwd_16traj()
    lens = np.diff(w.cu_seqlens)
    _, cost, _, _ = bca.pack_balanced(lens, w.s_copies, w.block_size, 8)
    rng = np.random.default_rng(5)
    B = 64
    prefix = B * rng.integers(16, 129, size=10000)
    copies = rng.integers(4, 25, size=10000)
    t0 = time.perf_counter()
    _, cost_big, _, _ = bca.pack_balanced(prefix + copies * B, copies, B, 64)
    pack_us = (time.perf_counter() - t0) * 1e6
    return {"workload": "16 trajectories into 8 bins; 10,000 random trajectories into 64 bins",
            "max_over_mean_cost_16traj_8bins": round(float(cost.max() / cost.mean()), 4),
            "max_over_mean_cost_10k_64bins": round(float(cost_big.max() / cost_big.mean()), 6),
            "host_us_10k_trajectories": round(pack_us, 1)}


def measured_peaks(probe: Probe, flush):
    """The machine's own peaks: dense bf16 MFMA rate with the clock it ran at,
    streaming read of 1 GiB, a cold read of 34 MB (the P = 8192 decode's
    bytes) and the event-timed empty kernel; then what the attention kernels'
    ingredients cost: MFMAs with 1 KB of LDS reads per wave for every MFMA
    (as in the kernels) or every second one, with the clock each ran at, and
    the issue cycles of v_fma_f32 and v_exp_f32 and of MFMAs with
    exponentials between them."""
    import torch
    out = torch.zeros(512 * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * 512, dtype=torch.int64, device="cuda")
    wgs, iters = 512, 4000

    def clock_mhz() -> float:
        # median over the workgroups of shader cycles per 100 MHz tick
        c = clk.cpu().view(-1, 2).double()
        return float(torch.median(c[:, 0] / c[:, 1].clamp(min=1)) * 100.0)

    def mfma():
        rc = probe.L.bca_probe_mfma(iters, wgs, ctypes.c_void_p(out.data_ptr()),
                                    ctypes.c_void_p(clk.data_ptr()), probe.stream())
        if rc != 0:
            raise RuntimeError("probe launch failed")

    per, _ = timed_calls(mfma, 5, 2)
    t_ms = statistics.median(per)
    mfma_mhz = clock_mhz()
    tflops = wgs * 4 * iters * 8 * 32768 / (t_ms * 1e-3) / 1e12
    big = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    per, _ = timed_calls(lambda: probe.read(big, 1 << 30, 256), 5, 2)
    read_1g = (1 << 30) / (statistics.median(per) * 1e-3) / 1e9
    per, _ = timed_calls(lambda: probe.read(big, 34213888, 2048), 15, 2, flush=flush)
    cold_us = statistics.median(per) * 1e3
    per, _ = timed_calls(probe.empty, 32, 3, flush=flush)
    empty_us = statistics.median(per) * 1e3

    # MFMA with the attention kernels' operand traffic: a 16-byte LDS read
    # per lane (1 KB per wave) before every MFMA, or before every second one
    out8 = torch.zeros(512 * 512, dtype=torch.float32, device="cuda")
    lds = {}
    for every, label in ((1, "1KB"), (2, "512B")):
        def run_lds():
            if probe.L.bca_probe_mfma_lds(1000, 512, every, ctypes.c_void_p(out8.data_ptr()),
                                          ctypes.c_void_p(clk.data_ptr()), probe.stream()) != 0:
                raise RuntimeError("probe launch failed")
        per, _ = timed_calls(run_lds, 5, 2)
        lds[label] = (512 * 8 * 1000 * 8 * 32768 / (statistics.median(per) * 1e-3) / 1e12,
                      clock_mhz())
    # VALU issue cost, cycles per wave-iteration on one SIMD: 16 v_exp_f32
    # (each after a v_mul_f32), 64 v_fma_f32, 8 MFMAs with the 16 v_exp_f32
    n_simd = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    valu = {}
    for kind in (0, 1, 2):
        def run_valu():
            if probe.L.bca_probe_valu(kind, 2000, 512, ctypes.c_void_p(out8.data_ptr()),
                                      ctypes.c_void_p(clk.data_ptr()), probe.stream()) != 0:
                raise RuntimeError("probe launch failed")
        per, _ = timed_calls(run_valu, 5, 2)
        cycles = statistics.median(per) * 1e-3 * clock_mhz() * 1e6
        valu[kind] = cycles / (512 * 8 * 2000 / n_simd)
    fma_cyc = valu[1] / 64
    return {"mfma_bf16_TFLOPs": round(tflops, 1),
            "mfma_frac_of_spec": round(tflops / PEAK_BF16_TFLOPS, 4),
            "clock_MHz_under_mfma": round(mfma_mhz, 0),
            "hbm_read_1GiB_GBps": round(read_1g, 1),
            "hbm_read_1GiB_frac_of_spec": round(read_1g / PEAK_HBM_GBS, 4),
            "read_34MB_after_512MB_flush_us_events": round(cold_us, 2),
            "empty_kernel_after_flush_us_events": round(empty_us, 2),
            "mfma_with_1KB_lds_read_each_TFLOPs": round(lds["1KB"][0], 1),
            "mfma_with_1KB_lds_read_each_clock_MHz": round(lds["1KB"][1], 0),
            "mfma_with_1KB_lds_read_per_2_TFLOPs": round(lds["512B"][0], 1),
            "mfma_with_1KB_lds_read_per_2_clock_MHz": round(lds["512B"][1], 0),
            "v_fma_f32_cycles_per_wave": round(fma_cyc, 2),
            "v_exp_f32_cycles_per_wave": round((valu[0] - 16 * fma_cyc) / 16, 2),
            "mfma_plus_exp_cycles_per_8_mfma": round(valu[2], 1)}


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default is all cores
        threads = os.cpu_count() or 1
    return model, int(threads)


def cpu_baseline(budget_s: float = 12.0):
    """The fp64 oracle (as it stands) on bounded samples, host BLAS threads.

    Headline: forward + backward of whole trajectories of the 16-trajectory
    staircase for KV head 0 and its four query heads (shortest trajectories
    first) until the budget is spent; useful FLOPs as on the GPU (14 * d per
    admitted pair per query head).  ``per_config``: a bounded sample of every
    other workload, each stated."""
    import numpy as np
    import oracle
    from block_diffusion_lm_causal_amd import workloads
    model, threads = cpu_info()
    w = workloads.staircase_bwd_16traj()
    lens = np.diff(w.cu_seqlens)
    grp = w.hq // w.hkv
    done, flops = [], 0.0
    t0 = time.perf_counter()
    for s in np.argsort(lens):
        a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        oracle.attention_bwd(w.q[a:b, :grp], w.k[a:b, :1], w.v[a:b, :1], w.do[a:b, :grp],
                             [0, b - a], [int(w.s_copies[s])], w.block_size, w.scale)
        pairs = workloads.useful_pairs([b - a], [int(w.s_copies[s])], w.block_size)
        flops += 14.0 * w.d * pairs * grp
        done.append(int(b - a))
        if time.perf_counter() - t0 > budget_s:
            break
    elapsed = time.perf_counter() - t0
    per_config = cpu_per_config()
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": model, "logical_cpus": os.cpu_count(),
            "sample": f"forward + backward of {len(done)} whole trajectories (L = "
                      f"{', '.join(map(str, done))}) of {HEADLINE}, KV head 0 with its "
                      f"{grp} query heads, {elapsed:.1f} s, fp64 numpy",
            "per_config": per_config}


def cpu_per_config():
    """Bounded oracle timings of the other workloads: median of 3 for the small
    ones (fp32 L=256, prefill KV head 0, decode), one run for the staircase."""
    import numpy as np
    import oracle
    from block_diffusion_lm_causal_amd import workloads

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    res = {}
    w = workloads.blockcausal_fp32_small()
    pairs = workloads.useful_pairs(np.diff(w.cu_seqlens), w.s_copies, w.block_size)
    t = timed(lambda: oracle.attention_fwd(w.q, w.k, w.v, w.cu_seqlens, None, w.block_size,
                                           w.scale), 3)
    res[w.name] = {"s": round(t, 4), "GFLOPs": round(4 * w.d * pairs * w.hq / t / 1e9, 2),
                   "sample": "whole workload, median of 3"}
    w = workloads.prefill_bf16_4k()
    pairs = workloads.useful_pairs(np.diff(w.cu_seqlens), w.s_copies, w.block_size)
    grp = w.hq // w.hkv
    t = timed(lambda: oracle.attention_fwd(w.q, w.k, w.v, w.cu_seqlens, None, w.block_size,
                                           w.scale, heads=list(range(grp))), 3)
    res[w.name] = {"s": round(t, 4), "GFLOPs": round(4 * w.d * pairs * grp / t / 1e9, 2),
                   "sample": f"query heads 0-{grp - 1} (KV head 0), all 4096 rows, median of 3"}
    for P in (1024, 8192):
        w = workloads.decode_step(P)
        t = timed(lambda: oracle.decode(w.q, w.k, w.v, w.scale), 3)
        flops = 4 * w.d * w.block_size * (P + w.block_size) * w.hq
        res[w.name] = {"s": round(t, 4), "GFLOPs": round(flops / t / 1e9, 2),
                       "sample": "whole step, median of 3"}
    w = workloads.staircase_fwd_8traj()
    lens = np.diff(w.cu_seqlens)
    s = int(np.argmin(lens))
    a, b = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
    t = timed(lambda: oracle.attention_fwd(w.q[a:b], w.k[a:b], w.v[a:b], [0, b - a],
                                           [int(w.s_copies[s])], w.block_size, w.scale), 1)
    pairs = workloads.useful_pairs([b - a], [int(w.s_copies[s])], w.block_size)
    res[w.name] = {"s": round(t, 4), "GFLOPs": round(4 * w.d * pairs * w.hq / t / 1e9, 2),
                   "sample": f"the shortest trajectory (L = {b - a}), all 32 heads, one run"}
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--skip-headline", action="store_true",
                    help="do not time the headline step (profiling runs of other paths)")
    ap.add_argument("--paths", default=ALL_PATHS,
                    help=f"comma list of extra paths to time (default {ALL_PATHS}; '' for none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (a known-size "
                         "kernel against which HBM byte counters are scaled)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_launch": nbytes,
                                               "bytes_written_per_launch": nbytes,
                                               "launches": 5}}), flush=True)
        return 0
    from block_diffusion_lm_causal_amd import bca, workloads
    bca.lib()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda", 0)
    extra = set(p for p in args.paths.split(",") if p)
    probe = Probe() if extra & {"decode", "decode_calls", "decode_splits", "peaks"} else None
    flush = flush_read = None
    if probe is not None:
        _flush_buf, flush_read = make_flush(dev, probe)
        flush = flush_read

    out = {"metric": "useful attention TFLOP/s (% bf16 MFMA peak); decode-step GB/s (% HBM peak)"}
    if not args.skip_headline:
        log("[bench] staircase forward + backward, 16 trajectories (headline)")
        w, pairs, kms, wall, step_ms = bench_headline(args.steps, args.warmup)
        ms_per_step = wall / args.steps
        fwd_flops = 4.0 * w.d * pairs * w.hq
        bwd_flops = 10.0 * w.d * pairs * w.hq
        dkdv_flops = 8.0 * w.d * pairs * w.hq
        value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12
        bwd_ms = step_ms["bwd"]
        achieved = dkdv_flops / (kms["bwd_dkdv_pp_kernel<128>"] * 1e-3) / 1e12
        out.update({
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": HEADLINE, "trajectories": w.nseq, "block_size": w.block_size,
                       "hq": w.hq, "hkv": w.hkv, "head_dim": w.d, "total_tokens": w.total,
                       "useful_pairs_per_head": pairs,
                       "flops_per_step": fwd_flops + bwd_flops,
                       "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
                       "fwd_ms": round(step_ms["fwd"], 4),
                       "fwd_frac_mfma": round(fwd_flops / step_ms["fwd"] / 1e9
                                              / PEAK_BF16_TFLOPS, 4),
                       "bwd_ms": round(bwd_ms, 4),
                       "bwd_frac_mfma_10d": round(bwd_flops / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                       "bwd_note": "bwd_ms: the whole backward call; kernel_ms_mean_events: "
                                   "each kernel launched on its own",
                       "kernel_ms_mean_events": {k: round(v, 4) for k, v in kms.items()}},
            "roofline": {"bound": "mfma", "kernel": "bwd_dkdv_pp_kernel<128>",
                         "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                         "traffic": stored_traffic("bwd_dkdv_16traj_B64")},
        })
    paths = {}
    if "peaks" in extra:
        log("[bench] measured peaks")
        out["measured_peaks"] = measured_peaks(probe, flush)
        if "roofline" in out:
            mp = out["measured_peaks"]["mfma_bf16_TFLOPs"]
            out["roofline"]["measured_peak"] = mp
            out["roofline"]["frac_of_measured_peak"] = round(out["roofline"]["achieved"] / mp, 4)
    if "prefill" in extra:
        log("[bench] block-causal prefill forward, 4096 tokens")
        paths["prefill_L4096"] = bench_prefill(max(args.steps, 20), args.warmup)
    if "decode_calls" in extra:  # flushed calls only (short runs under the profilers)
        for P in (1024, 8192):
            log(f"[bench] decode P={P}, flushed calls only")
            paths[f"decode_P{P}_calls"] = bench_decode_calls(P, flush)
    if "decode_splits" in extra:  # split-count sweep (not in the default run)
        log("[bench] decode split-count sweep")
        paths["decode_splits"] = bench_decode_splits(flush)
    if "decode" in extra:
        for P in (1024, 8192):
            log(f"[bench] decode P={P}")
            paths[f"decode_P{P}"] = bench_decode(P, probe, flush, flush_read)
        for P in (1024, 8192):
            log(f"[bench] decode, FP8 cache, P={P}")
            paths[f"decode_fp8_P{P}"] = bench_decode(P, probe, flush, flush_read, fp8=True)
    if "groups" in extra:
        log("[bench] general staircase (copy groups), forward + backward, 8 trajectories")
        paths["staircase_groups_fwdbwd_8traj"] = bench_groups(10, 3)
    if "packing" in extra:
        paths["packing"] = bench_packing()
    if "staircase" in extra:
        log("[bench] staircase forward, 8 trajectories")
        paths["staircase_fwd_8traj"] = bench_staircase8(max(5, args.steps // 2), 3)
    out["paths"] = paths
    if not args.skip_cpu:
        log("[bench] CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
