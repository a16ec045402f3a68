"""The C ABI's argument checks under host AddressSanitizer (CPU only).

exact_attention_66_amd.asan_build compiles attn_api.cpp and attn_profile.cpp
with host AddressSanitizer and links them with the regular kernel objects;
the ABI tests (tests/test_abi.py: every rejection path, the workspace
arithmetic, the exported symbols) then run in a subprocess against that
library with the sanitizer runtime preloaded.  Any invalid read or write in
the checking code ends that run with an AddressSanitizer report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_abi_checks_clean_under_host_asan():
    from exact_attention_66_amd import asan_build, build

    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    if not all(os.path.exists(os.path.join(build.BUILD_DIR, s + ".o")) for s in build.SOURCES):
        build.build()
    lib = asan_build.build_asan()
    rt = asan_build.runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, ATTN_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               HIP_VISIBLE_DEVICES="")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout
