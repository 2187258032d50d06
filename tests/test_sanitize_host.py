"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU).  bca_api.cpp, bca_pack.cpp and a driver (abi_sanitize_driver.cpp)
are compiled for the host with g++ and the sanitizers, linked with the kernel
objects of the normal build (only their host-side launchers are reachable, and
no call in the driver gets that far), and run: every validation path of every
entry point and the packing routines on random host data."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_diffusion_lm_causal_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
KERNEL_OBJECTS = ("attn_fwd_bf16.o", "attn_decode_bf16.o", "attn_fwd_f32.o", "attn_bwd_bf16.o",
                  "bca_util.o", "bca_scratch.o")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def test_c_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJECTS]
    if gxx is None or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs g++ and the built kernel objects (python -m "
                    "block_diffusion_lm_causal_amd.build)")
    flags = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"] + SAN
    mine = []
    for src in (os.path.join(CSRC, "bca_api.cpp"), os.path.join(CSRC, "bca_pack.cpp"),
                os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([gxx, *flags, "-c", src, "-o", o], check=True, capture_output=True,
                       text=True)
        mine.append(o)
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run([gxx, *SAN, *mine, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True, capture_output=True,
                   text=True)
    # verify_asan_link_order=0: the environment may preload other libraries
    # ahead of the sanitizer runtime; they are left as they are.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-4000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "ok: 0 failed" in r.stdout
