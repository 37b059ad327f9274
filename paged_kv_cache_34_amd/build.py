"""Build the HIP library `libpaged_attn.so` for gfx950 with hipcc.

Usage: python -m paged_kv_cache_34_amd.build   (or build() from Python)

Each translation unit under csrc/ is compiled in parallel into _build/, then
linked into paged_kv_cache_34_amd/libpaged_attn.so next to this file.  All
device code is built with packed-fp32 instructions disabled.  Extra hipcc
flags may be given in the environment variable PA_HIPCC_FLAGS (whitespace
separated), e.g. the compile-time tuning macros of csrc/decode_kernels.h
(PA_DECODE_DEPTH, PA_DECODE_DEPTH_FP8, PA_DECODE_PERSIST_PER_CU,
PA_FP8_FEW_ITEMS_PERSIST_PER_CU) to reproduce the variants those macros
document.
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
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libpaged_attn.so")
SOURCES = ["api.hip", "decode.hip", "decode_fp8.hip", "decode_xpacked.hip", "decode_tokens.hip", "prefill.hip", "kvcache.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")
    return path


def _flags():
    # -amdgpu-mfma-vgpr-form: MFMA accumulators in arch VGPRs.  With the
    # default AGPR form the decode tile loop copied all its PV accumulators
    # AGPR -> VGPR on every iteration (for the rarely taken softmax rescale),
    # about a third of its vector ALU work, and the FP8 decode kernels needed
    # more registers (D=256: one wave per SIMD instead of two).
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"] + \
        os.environ.get("PA_HIPCC_FLAGS", "").split()


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{proc.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}", file=sys.stderr)
    return LIBRARY


if __name__ == "__main__":
    build()
