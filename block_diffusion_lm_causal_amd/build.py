"""Build libbca.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m block_diffusion_lm_causal_amd.build`` (or ``build()`` from
Python).  Every source is compiled on every call; objects go to ``_build/``
next to this file and the shared library to ``libbca.so`` in the package.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbca.so")
PROBE_LIB = os.path.join(PKG, "libbca_probe.so")  # machine microbenchmarks (bench.py only)
ARCH = "gfx950"

SOURCES = [
    "bca_api.cpp",
    "bca_pack.cpp",
    "attn_fwd_bf16.hip",
    "attn_decode_bf16.hip",
    "attn_fwd_f32.hip",
    "attn_bwd_bf16.hip",
    "bca_util.hip",
    "bca_scratch.hip",
]
PROBE_SOURCES = ["probe.hip"]

# Packed fp32 VALU forms are disabled: the compiler emits plain fp32 ops.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    # No NaN reaches the kernels' max/compare chains (masked scores are -inf), so
    # the compiler need not canonicalise MFMA results before every fmaxf.
    "-fno-honor-nans",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbca.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link libbca.so (and the microbenchmark library
    libbca_probe.so); returns the path of libbca.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
