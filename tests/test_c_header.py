"""The boundary from C: include/attn.h compiles as strict C99 and as C++17, and a C program links
against libattn.so and calls it (host-side calls only: version, status strings, size queries
and argument rejections, none of which touches a GPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "transformer_self_attention_amd")
ROCM_LIB = "/opt/rocm/lib"

PROGRAM = r"""
#include <stdio.h>
#include "attn.h"

int main(void) {
  static float table[16];
  int32_t pos[2] = {0, 0};
  printf("version %d\n", attn_version());
  printf("ok %s\n", attn_status_string(ATTN_OK));
  printf("invalid %s\n", attn_status_string(ATTN_ERR_INVALID_ARG));
  printf("table_bytes %lu\n", (unsigned long)attn_rope_table_bytes(8192, 128));
  printf("prefill_ws %lu\n", (unsigned long)attn_prefill_workspace_bytes(1, 8, 8192, 128));
  printf("decode_splits %d\n", attn_decode_num_splits(32, 64, 8, 8192, 128, 0));
  /* rejected on the host before any device call */
  printf("prefill_null %d\n", (int)attn_prefill(NULL, NULL, NULL, NULL, NULL, ATTN_BF16, ATTN_BF16, 1, 8, 2, 64,
                                                 128, 1, 0, -1, table, 64, NULL, 0, NULL));
  printf("append_null %d\n", (int)attn_cache_append(NULL, NULL, NULL, NULL, pos, 2, 2, 1, 64, 128, NULL, 0, NULL));
  printf("checked %d\n", attn_checked_sites(NULL, 0));
  return 0;
}
"""


def _compiler(name):
    path = shutil.which(name)
    if not path:
        pytest.skip(f"{name} not available")
    return path


def _lib():
    lib = os.path.join(PKG, "libattn.so")
    if not os.path.exists(lib):
        pytest.skip("libattn.so is not built")
    return lib


def test_header_compiles_as_strict_c99_and_cpp17(tmp_path):
    src_c = tmp_path / "h.c"
    src_c.write_text('#include "attn.h"\nint use(void) { return attn_version(); }\n')
    subprocess.run([_compiler("gcc"), "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, "-c",
                    str(src_c), "-o", str(tmp_path / "h.o")], check=True, capture_output=True)
    src_cc = tmp_path / "h.cc"
    src_cc.write_text('#include "attn.h"\nint use() { return attn_version(); }\n')
    subprocess.run([_compiler("g++"), "-std=c++17", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE, "-c",
                    str(src_cc), "-o", str(tmp_path / "hh.o")], check=True, capture_output=True)


def test_c_program_links_and_calls_the_library(tmp_path):
    _lib()
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    r = subprocess.run([_compiler("gcc"), "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE, str(src), "-o",
                        str(exe), "-L", PKG, "-lattn", f"-Wl,-rpath,{PKG}", "-L", ROCM_LIB, f"-Wl,-rpath,{ROCM_LIB}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr[-2000:]
    got = dict(line.split(" ", 1) for line in out.stdout.strip().splitlines())
    from transformer_self_attention_amd import lib
    assert int(got["version"]) == lib.version()
    assert got["ok"] == "ATTN_OK" and got["invalid"].startswith("ATTN_ERR_")
    assert int(got["table_bytes"]) == 8192 * 128 * 4
    assert int(got["prefill_ws"]) == lib.prefill_workspace_bytes(1, 8, 8192, 128)
    assert int(got["decode_splits"]) == lib.decode_num_splits(32, 64, 8, 8192, 128, 0)
    assert int(got["prefill_null"]) == lib.ATTN_ERR_INVALID_ARG
    assert int(got["append_null"]) == lib.ATTN_ERR_INVALID_ARG
    assert int(got["checked"]) == -1
