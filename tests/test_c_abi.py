"""The header is plain C and the library links from C without Python.

A small C99 program that includes include/dsa_sparse_mla.h is compiled with
gcc -Wall -Werror, linked against the built library, and run. It calls only
host-side paths (version, status strings, argument validation that returns
before any HIP call), so it needs no GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "dsa_sparse_mla_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "dsa_sparse_mla.h"

int main(void) {
  int bad = 0;
  if (dsa_version() < 100) bad |= 1;
  if (strcmp(dsa_status_string(DSA_OK), "ok") != 0) bad |= 2;
  /* an empty batch is a no-op */
  if (dsa_sparse_mla_fwd(0, 0, 0, 0, 0, 0, 0, 0, /*T*/ 0, 8, 2048, 0.04f, 0, 0, 0, 0, 0, 0, 0, 0, 0) != DSA_OK)
    bad |= 4;
  /* a null q with tokens is rejected on the host */
  if (dsa_sparse_mla_fwd(0, 576, 576, 0, 576, 10, 0, 2048, 4, 8, 2048, 0.04f, 0, 512, 512, 0, 8, 0, 0, 0, 0)
      != DSA_ERR_INVALID_ARGUMENT)
    bad |= 8;
  /* unsupported head count, before any pointer is looked at */
  if (dsa_sparse_mla_bwd(0, 0, 0, 0, 0, 0, 0, 0, 4, 129, 2048, 0.04f, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0,
                         0, 0) != DSA_ERR_UNSUPPORTED)
    bad |= 16;
  int32_t sched = -1;
  int64_t bwd_bytes = -1;
  if (dsa_sparse_mla_bwd_workspace_size(2119, 8, 2119, 2048, &sched, &bwd_bytes) != DSA_OK ||
      sched != DSA_BWD_KV_MAJOR || bwd_bytes <= 0)
    bad |= 64;
  int32_t splits = -1;
  int64_t bytes = -1;
  if (dsa_sparse_mla_workspace_size(100, 8, 2048, 1, &splits, &bytes) != DSA_OK || splits != 1 || bytes != 0)
    bad |= 32;
  printf("c abi %s (%d)\n", bad ? "FAILED" : "ok", bad);
  return bad;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_compiles_as_c_and_links(tmp_path):
    lib = os.path.join(LIBDIR, "libdsa_sparse_mla.so")
    if not os.path.exists(lib):
        pytest.skip("library not built")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", LIBDIR, "-ldsa_sparse_mla",
                    f"-Wl,-rpath,{LIBDIR}"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "c abi ok" in res.stdout
