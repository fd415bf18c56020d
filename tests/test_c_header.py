"""The C ABI from C: a small C11 program includes include/apbv.h, links libapbv.so and calls
the host-only entry points and a validation error (no GPU work; runs on the CPU)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import sequence_approximate_attention_score_amd as apbv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sequence_approximate_attention_score_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "apbv.h"

int main(void) {
  /* 4 blocks of 1024 rows: 2 ZigZag buckets, 4 tiles of 256 rows per block */
  int32_t bs[5] = {0, 1024, 2048, 3072, 4096};
  apbv_layout lay;
  memset(&lay, 0, sizeof(lay));
  lay.n_blocks = 4;
  lay.block_starts = bs;
  lay.l_anchor = 128;
  lay.l_query = 64;
  lay.l_pass = 128;
  lay.hq = 28;
  lay.hkv = 4;
  lay.head_dim = 128;
  lay.zigzag = 1;
  int32_t units = 0;
  size_t ws = 0;
  const apbv_status s1 = apbv_schedule(&lay, 0, 0, NULL, 0, &units);
  const apbv_status s2 = apbv_score_select_workspace(&lay, &ws);
  printf("version %s\n", apbv_version());
  printf("tile_rows %d buckets %d units %d status %d %d workspace %zu\n",
         apbv_attn_tile_rows(128), apbv_num_buckets(&lay), units, s1, s2, ws);
  lay.head_dim = 96;   /* not implemented: refused before anything is launched */
  const apbv_status s3 = apbv_approx_attn_prefill(&lay, NULL, NULL, NULL, NULL, NULL, NULL,
                                                  NULL, 0, 0, NULL);
  printf("head_dim 96: %s (%s)\n", apbv_status_str(s3), apbv_last_error());
  return s3 == APBV_EUNSUPPORTED ? 0 : 1;
}
"""


def test_header_compiles_as_c_and_the_library_links(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    apbv.lib()   # the library is built
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    os.path.join(PKG, "libapbv.so"), f"-Wl,-rpath,{PKG}"],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert lines[0].startswith("version apbv-gfx950")
    # 2 buckets of 4 units: unit t pairs tile t of one block with tile 3 - t of the other
    assert lines[1].startswith("tile_rows 256 buckets 2 units 8 status 0 0 workspace ")
    assert int(lines[1].split()[-1]) > 0
    assert "head_dim = 96" in lines[2] and "unsupported" in lines[2].lower()
