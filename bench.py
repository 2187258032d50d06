#!/usr/bin/env python3
"""Benchmark of block-causal / staircase attention on one MI355X.

Headline (``value``): useful TFLOP/s of the block-causal prefill forward on
one 4096-token sequence, 32 query heads sharing 8 KV heads, head_dim 128,
block size 32, bf16 (4 * d FLOPs per admitted query-key pair per query head;
masked pairs and padded tiles are not counted).  One step is one call of the
forward over that whole input, inputs resident in HBM.

The same run also measures the other cases of the path and reports them
under ``"paths"``:
  * decode step, 32 queries against a prefix of 1024 or 8192 keys plus the
    block's own 32 (GQA 32/8, d 128): HBM GB/s of the algorithmic bytes
    (K and V read once per KV head, Q read, O and LSE written), median over
    32 calls with L2 and the Infinity Cache flushed (by reading 512 MB)
    before each call, plus the
    warm back-to-back figure and the per-step time of a captured 32-step
    graph (caches warm), labelled; the same against an FP8 E4M3 cache;
  * staircase forward, 8 packed trajectories (block 32);
  * staircase forward and backward, 16 packed trajectories (block 64),
    backward FLOPs counted as 10 * d per admitted pair per query head;
  * the general trajectory staircase (a group of copies per block), forward
    and backward, 8 trajectories (block 32);
  * compute-balanced packing of trajectories into bins (host routine).

``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the
headline workload (whole query heads until about 10 s have elapsed).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-cpu]
       [--only-headline] [--paths decode,staircase,groups,packing] [--copy-calibration]
Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
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
CSRC = os.path.join(ROOT, "block_diffusion_lm_causal_amd", "csrc")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# Sources the headline forward kernel is built from.
FWD_SOURCES = ("attn_fwd_bf16.hip", "attn_common.hpp", "bca_device.hpp", "bca_kernels.hpp")


def source_digest(files=FWD_SOURCES) -> str:
    """Hash of a kernel's sources: stored HBM-traffic counters are used only
    while that kernel is unchanged."""
    h = hashlib.sha256()
    for name in sorted(files):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_tag: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken with the current kernel sources (else None)."""
    path = os.path.join(PROFILES, f"{kernel_tag}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != source_digest():
        return None
    return float(m_val.group(1))


def timed_calls(fn, steps: int, warmup: int, flush=None):
    """Run fn() warmup + steps times; returns (per-call event ms list, wall ms of the
    timed region).  With flush, the cache flush runs before every timed call,
    outside its events, and the wall figure is not meaningful."""
    import torch
    # W warm-up calls, continued until about a second of work has run so the GPU
    # clocks have settled before the timed region.
    t_warm = time.perf_counter()
    done = 0
    while done < warmup or (time.perf_counter() - t_warm < 1.0 and done < 20 * max(warmup, 1)):
        fn()
        done += 1
        if done % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
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
    return w, flops, per_call, wall


def make_flush(dev):
    """Evict L2 and the Infinity Cache before a timed call by READING 512 MB
    (a decode loop streams the model's weights between steps).  A write-based
    flush would leave dirty lines whose write-back competes with the call."""
    import torch
    buf = torch.zeros(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros((), dtype=torch.float32, device=dev)
    return lambda: sink.copy_(buf.sum())


def bench_decode(prefix: int, calls: int = 32):
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    w = workloads.decode_step(prefix)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (w.q, w.k, w.v))
    ws_bytes = bca.decode_workspace(w.block_size, prefix + w.block_size, w.hq, w.hkv, w.d)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.block_size), dtype=torch.float32, device=dev)
    kv_len = prefix + w.block_size
    algo_bytes = (2 * kv_len * w.hkv * w.d * 2 + 2 * w.block_size * w.hq * w.d * 2
                  + w.hq * w.block_size * 4)
    flush = make_flush(dev)

    def step():
        bca.decode(q, k, v, w.scale, workspace=ws, out=o, lse=lse)

    cold, _ = timed_calls(step, calls, 3, flush=flush)
    warm, _ = timed_calls(step, calls, 3)
    cold_us = statistics.median(cold) * 1e3
    warm_us = statistics.median(warm) * 1e3
    # the denoising loop of one block as one captured graph of `calls` steps
    graph = bca.DecodeGraph(q, k, v, calls, w.scale, workspace=ws, out=o, lse=lse)
    replays, _ = timed_calls(graph.launch, 10, 2)
    graph.close()
    graph_us = statistics.median(replays) * 1e3 / calls
    return {
        "workload": w.name, "bytes_per_call": algo_bytes,
        "us_per_call_flushed_median": round(cold_us, 3),
        "GBps_flushed": round(algo_bytes / cold_us / 1e3, 1),
        "frac_hbm_flushed": round(algo_bytes / cold_us / 1e3 / PEAK_HBM_GBS, 4),
        "us_per_call_warm_median": round(warm_us, 3),
        "GBps_warm_l2_resident": round(algo_bytes / warm_us / 1e3, 1),
        "us_per_step_graph_replay": round(graph_us, 3),
        "GBps_graph_replay_l2_resident": round(algo_bytes / graph_us / 1e3, 1),
        "calls": calls,
    }


def bench_decode_fp8(prefix: int, calls: int = 32):
    """Decode step against an FP8 E4M3 cache: K/V bytes halve."""
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    w, k8, v8, ks, vs = workloads.decode_step_fp8(prefix)
    dev = torch.device("cuda", 0)
    q, k8, v8 = w.q.to(dev), k8.to(dev), v8.to(dev)
    kv_len = prefix + w.block_size
    ws = torch.empty(max(bca.decode_workspace(w.block_size, kv_len, w.hq, w.hkv, w.d), 16),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.hq, w.block_size), dtype=torch.float32, device=dev)
    algo_bytes = (2 * kv_len * w.hkv * w.d + 2 * w.block_size * w.hq * w.d * 2
                  + w.hq * w.block_size * 4)
    flush = make_flush(dev)

    def step():
        bca.decode_fp8(q, k8, v8, ks, vs, w.scale, workspace=ws, out=o, lse=lse)

    cold, _ = timed_calls(step, calls, 3, flush=flush)
    warm, _ = timed_calls(step, calls, 3)
    cold_us = statistics.median(cold) * 1e3
    warm_us = statistics.median(warm) * 1e3
    return {"workload": w.name, "bytes_per_call": algo_bytes,
            "us_per_call_flushed_median": round(cold_us, 3),
            "GBps_flushed": round(algo_bytes / cold_us / 1e3, 1),
            "frac_hbm_flushed": round(algo_bytes / cold_us / 1e3 / PEAK_HBM_GBS, 4),
            "us_per_call_warm_median": round(warm_us, 3), "calls": calls}


def bench_staircase(workload_fn, steps: int, warmup: int, backward: bool):
    import numpy as np
    import torch
    from block_diffusion_lm_causal_amd import bca, workloads
    w = workload_fn()
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
    res = {"workload": w.name, "total_tokens": w.total, "useful_pairs_per_head": pairs,
           "fwd_ms_median": round(fwd_ms, 4),
           "fwd_TFLOPs": round(fwd_flops / fwd_ms / 1e9, 1),
           "fwd_frac_mfma": round(fwd_flops / fwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4)}
    if backward:
        do = w.do.to(dev)
        ws = torch.empty(bca.staircase_bwd_workspace(w.total, w.hq, w.hkv, w.d),
                         dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fwd()

        def bwd():
            bca.staircase_bwd(q, k, v, o, lse, do, cu, sc, w.block_size, w.scale, w.max_seqlen,
                              workspace=ws, dq=dq, dk=dk, dv=dv)

        per_call, _ = timed_calls(bwd, steps, warmup)
        bwd_ms = statistics.median(per_call)
        bwd_flops = 10.0 * w.d * pairs * w.hq
        res.update({"bwd_ms_median": round(bwd_ms, 4),
                    "bwd_TFLOPs_10d": round(bwd_flops / bwd_ms / 1e9, 1),
                    "bwd_frac_mfma_10d": round(bwd_flops / bwd_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                    "bwd_TFLOPs_4d": round(0.4 * bwd_flops / bwd_ms / 1e9, 1)})
    return res


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


def cpu_baseline(budget_s: float = 10.0):
    """The fp64 oracle on whole query heads of the headline workload until the
    budget is spent (at least one head)."""
    import numpy as np
    import oracle
    from block_diffusion_lm_causal_amd import workloads
    w = workloads.prefill_bf16_4k()
    pairs = workloads.useful_pairs(np.diff(w.cu_seqlens), w.s_copies, w.block_size)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default is all cores
        cores = os.cpu_count() or 1
    heads = 0
    t0 = time.perf_counter()
    while heads < w.hq and (heads == 0 or time.perf_counter() - t0 < budget_s):
        oracle.attention_fwd(w.q, w.k, w.v, w.cu_seqlens, None, w.block_size, w.scale,
                             heads=[heads])
        heads += 1
    elapsed = time.perf_counter() - t0
    flops = 4.0 * w.d * pairs * heads
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{heads} of {w.hq} query heads of {w.name} (all 4096 rows), "
                      f"{elapsed:.1f} s, fp64 numpy"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--only-headline", action="store_true", help="time the headline case only")
    ap.add_argument("--paths", default="decode,staircase,groups,packing",
                    help="comma list of extra paths to time: decode, staircase, groups, packing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (a known-size "
                         "kernel against which HBM byte counters are scaled)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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

    log("[bench] prefill forward (headline)")
    w, flops, per_call, wall = bench_prefill(args.steps, args.warmup)
    ms_per_step = wall / args.steps
    kernel_ms = statistics.mean(per_call)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    traffic = stored_traffic("fwd_bf16_prefill_L4096")

    paths = {}
    extra = set() if args.only_headline else set(p for p in args.paths.split(",") if p)
    if "decode" in extra:
        for P in (1024, 8192):
            log(f"[bench] decode P={P}")
            paths[f"decode_P{P}"] = bench_decode(P)
        for P in (1024, 8192):
            log(f"[bench] decode, FP8 cache, P={P}")
            paths[f"decode_fp8_P{P}"] = bench_decode_fp8(P)
    if "groups" in extra:
        log("[bench] general staircase (copy groups), forward + backward, 8 trajectories")
        paths["staircase_groups_fwdbwd_8traj"] = bench_groups(10, 3)
    if "packing" in extra:
        paths["packing"] = bench_packing()
    if "staircase" in extra:
        log("[bench] staircase forward, 8 trajectories")
        paths["staircase_fwd_8traj"] = bench_staircase(workloads.staircase_fwd_8traj,
                                                       max(5, args.steps // 5), 3, False)
        log("[bench] staircase forward + backward, 16 trajectories")
        paths["staircase_fwdbwd_16traj"] = bench_staircase(workloads.staircase_bwd_16traj,
                                                           5, 2, True)

    cpu = None
    if not args.skip_cpu:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline()

    out = {
        "metric": "useful attention TFLOP/s (% bf16 MFMA peak); decode-step GB/s (% HBM peak)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "seq_len": 4096, "block_size": 32, "hq": 32, "hkv": 8,
                   "head_dim": 128, "batch": 1, "kernel": "fwd_pp_kernel<128>",
                   "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "kernel_ms_mean": round(kernel_ms, 5),
        "paths": paths,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
