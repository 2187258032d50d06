"""Resource checks of every HIP kernel, from the gfx950 code object metadata
the compiler writes (no GPU needed): no kernel uses scratch memory or spills
registers, and each fits the 160 KB of LDS of a compute unit.

A kernel that indexes a register array with a run-time value, or needs more
registers than its launch bounds allow, is moved to scratch memory by the
compiler: its results stay correct, so only its speed would show it (a decode
kernel written that way ran 2.5 times slower).
"""
import concurrent.futures
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from block_diffusion_lm_causal_amd import build as B

LDS_BYTES = 160 * 1024
HIP_SOURCES = [s for s in B.SOURCES + B.PROBE_SOURCES if s.endswith(".hip")]


def _hipcc_or_skip() -> str:
    try:
        return B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available")


def _kernel_metadata(asm: str):
    """(name, private segment bytes, VGPR spills, SGPR spills, LDS bytes) per kernel."""
    out = []
    for block in re.split(r"\n\s+- \.(?=\w)", asm.split("amdhsa.kernels:", 1)[-1]):
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name or not re.search(r"\.private_segment_fixed_size:", block):
            continue

        def field(key):
            m = re.search(rf"\.{key}:\s+(\d+)", block)
            return int(m.group(1)) if m else None
        out.append((name.group(1), field("private_segment_fixed_size"),
                    field("vgpr_spill_count"), field("sgpr_spill_count"),
                    field("group_segment_fixed_size")))
    return out


@pytest.fixture(scope="module")
def kernels():
    cc = _hipcc_or_skip()
    tmp = tempfile.mkdtemp(prefix="bca_res_")

    def compile_one(src):
        out = os.path.join(tmp, src + ".s")
        cmd = [cc, *B.COMMON_FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src),
               "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            return src, _kernel_metadata(f.read())
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(HIP_SOURCES)) as ex:
            found = dict(ex.map(compile_one, HIP_SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return found


def test_every_source_has_kernels(kernels):
    for src in HIP_SOURCES:
        if src == "bca_scratch.hip":
            continue  # holds only the no-allocation entry point's device array
        assert kernels[src], f"no kernel metadata parsed from {src}"


def test_no_scratch_no_spills_lds_fits(kernels):
    bad = []
    for src, ks in kernels.items():
        for name, priv, vspill, sspill, lds in ks:
            if priv or vspill or sspill or (lds or 0) > LDS_BYTES:
                bad.append((src, name, priv, vspill, sspill, lds))
    assert not bad, bad
