"""Host-side AddressSanitizer build of the C ABI's argument checking (CPU only).

The validation code of attn_api.cpp and attn_profile.cpp is compiled with
host AddressSanitizer (``-Xarch_host`` before the sanitizer flag, so no GPU
code is instrumented) and linked with the kernel objects of the regular build
into ``_build/libattn_asan.so``.  tests/test_abi_asan.py loads that library
with the sanitizer runtime preloaded and runs the ABI tests against it: every
rejection path (null, shape, alignment, aliasing, layout, dropout, workspace)
runs under the sanitizer.  Never shipped and never run on a GPU.

Usage: python -m exact_attention_66_amd.asan_build   (after the regular build)
"""
from __future__ import annotations

import os
import subprocess
import sys

from . import build as B

ASAN_LIB = os.path.join(B.BUILD_DIR, "libattn_asan.so")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-fno-omit-frame-pointer", "-shared-libasan"]
VALIDATION_SOURCES = ["attn_api.cpp", "attn_profile.cpp"]


def runtime() -> str:
    """Path of the host AddressSanitizer runtime matching the compiler."""
    clang = os.path.join(os.path.dirname(os.path.realpath(B.HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def build_asan() -> str:
    os.makedirs(B.BUILD_DIR, exist_ok=True)
    objs = []
    for src in VALIDATION_SOURCES:
        obj = os.path.join(B.BUILD_DIR, "asan_" + src + ".o")
        cmd = [B.HIPCC, *B.COMMON, *HOST_ASAN, "-c", os.path.join(B.CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"asan compile of {src} failed:\n{res.stderr}")
        objs.append(obj)
    kernels = [os.path.join(B.BUILD_DIR, s + ".o") for s in B.SOURCES if s not in VALIDATION_SOURCES]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        raise RuntimeError(f"run the regular build first (missing {missing})")
    cmd = [B.HIPCC, *B.DEVICE, *HOST_ASAN, "-shared", "-fPIC", *objs, *kernels, "-o", ASAN_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"asan link failed:\n{res.stderr}")
    return ASAN_LIB


if __name__ == "__main__":
    print(build_asan())
    sys.exit(0)
