"""The public header is plain C: a C99 translation unit that includes it, calls
the host-only entry points and links against the built library compiles with
-Wall -Werror and runs (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "kv_cache_int2_amd")
LIB = os.path.join(LIB_DIR, "libkv_cache_int2_amd.so")

SRC = r"""
#include <stdio.h>
#include <string.h>
#include "oscar.h"

int main(int argc, char** argv) {
  oscar_shape s;
  memset(&s, 0, sizeof s);
  s.n_q_heads = 32; s.n_kv_heads = 8; s.head_dim = OSCAR_HEAD_DIM; s.group_size = 128;
  s.page_size = OSCAR_PAGE_SIZE; s.window = 128; s.n_sink = 0;
  if (OSCAR_BLOCK_BYTES_FOR_GROUP(128) != OSCAR_BLOCK_BYTES) return 1;
  if (OSCAR_BLOCK_BYTES_FOR_GROUP(32) != 1536) return 2;
  if (oscar_rotation_file_bytes(2, 8, 1) != 64 + 2 * (8 * 128 * 128 * 2 * 2 + 8 * 128 * 8 * 2)) return 3;
  if (strcmp(oscar_strerror(OSCAR_OK), "ok") != 0) return 4;
  if (oscar_rotation_read_info(argv[1], NULL, NULL, NULL, NULL) != OSCAR_EIO) return 5;
  s.group_size = 48;
  if (oscar_quantize_append(&s, 0, 0, 0, 0, 1, 0, 0, 1, 0, 1, 0, 0, 1, 0, 0, 0) != OSCAR_EUNSUPPORTED) return 6;
  puts("c-abi ok");
  (void)argc;
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists(LIB), reason="gcc or the library missing")
def test_header_compiles_as_c99_and_links(tmp_path):
    src = tmp_path / "demo.c"
    src.write_text(SRC)
    exe = tmp_path / "demo"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-L", LIB_DIR, "-lkv_cache_int2_amd", f"-Wl,-rpath,{LIB_DIR}", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe), str(tmp_path / "missing.oscarrot")], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c-abi ok" in r.stdout, (r.returncode, r.stdout, r.stderr)
