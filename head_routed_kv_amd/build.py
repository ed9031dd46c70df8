"""Build libheadcast.so for gfx950 with hipcc, in-tree.

    python -m head_routed_kv_amd.build          # the library
    python -m head_routed_kv_amd.build --asan   # host code under AddressSanitizer

Objects go to head_routed_kv_amd/_build/, the library to
head_routed_kv_amd/libheadcast.so.  The --asan build instruments the host
code only (argument checks, layout and planning; GPU code is built as
usual) into libheadcast_asan.so, for running the host-side tests:

    ASAN_OPTIONS=detect_leaks=0 LD_PRELOAD=$(hipcc -print-file-name=libclang_rt.asan-x86_64.so) \
        HEADCAST_LIB=head_routed_kv_amd/libheadcast_asan.so python -m pytest tests/test_abi.py
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libheadcast.so")
ASAN_LIB = os.path.join(PKG, "libheadcast_asan.so")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
SOURCES = ["api.hip", "append.hip", "attn_bf16.hip", "attn_f32.hip", "classify.hip"]
ARCH = os.environ.get("HEADCAST_ARCH", "gfx950")

# Packed fp32 VALU instructions stay off: the compiler otherwise forms them
# from ordinary float code.  MFMAs are selected in VGPR form: the attention
# kernel's softmax reads the score accumulators with VALU instructions, and the
# AGPR form made the register allocator copy every O accumulator between AGPRs
# and VGPRs on each key tile.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form=1",
               "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int = 5, asan: bool = False) -> str:
    out_dir = os.path.join(OUT_DIR, "asan") if asan else OUT_DIR
    lib = ASAN_LIB if asan else LIB
    extra = ASAN_FLAGS if asan else []
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()

    def one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = lib + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asan="--asan" in sys.argv))
