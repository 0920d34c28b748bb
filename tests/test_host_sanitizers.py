"""The launch layer's host code under AddressSanitizer and UBSan (CPU only).

Builds the library with the sanitizers on the host side only (every
-fsanitize flag follows -Xarch_host, so no device code is instrumented), then
runs the C ABI's host-validation tests (tests/test_abi.py) in a subprocess
that preloads the ASan runtime and loads that build (DSA_SPARSE_MLA_LIB). A
sanitizer report aborts the subprocess (halt_on_error), which fails this test.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asan_runtime():
    try:
        out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True, timeout=60).stdout.strip()
    except (OSError, subprocess.TimeoutExpired):
        return None
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_under_host_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime next to hipcc")
    lib = tmp_path / "libdsa_sparse_mla_asan.so"
    src = os.path.join(ROOT, "dsa_sparse_mla_amd", "csrc", "dsa_sparse_mla.hip")
    flags = ("--offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -shared "
             "-Xclang -target-feature -Xclang -packed-fp32-ops "
             "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-omit-frame-pointer -shared-libsan").split()
    cmd = [HIPCC, *flags, "-I", os.path.join(ROOT, "include"), "-I", os.path.dirname(src), src, "-o", str(lib)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "DSA_SPARSE_MLA_LIB": str(lib),
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    probe = ("import dsa_sparse_mla_amd as d; d.lib(); "
             "m = open('/proc/self/maps').read(); "
             f"assert {str(lib)!r} in m and 'libclang_rt.asan' in m, 'sanitized build not loaded'")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
