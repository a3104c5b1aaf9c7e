"""The C boundary used from C: a C99 program compiled with gcc against
include/lf.h (strict, warnings as errors) and linked to liblf.so calls the
host-only entry points and the validation path of a GPU entry point (no
device work), and checks their results.

Expected values: the rolling cache of 9 slots at chunk 4 of 3-frame chunks
holds absolute frames 6..14 in slots a mod 9; the rollout budget
(7 chunks, sigma linear 0.1..1, chunk 0 dense, s_base 0.9, mean 0.8)
solves beta = (s_base - s_target) * n / sum(1/sqrt(sigma_i)) over the six
non-dense chunks, recomputed here in Python from that closed form.
"""
import math
import os
import shutil
import subprocess

import pytest

from block_sparse_attention_lf_amd import lf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = r"""
#include <stdio.h>
#include "lf.h"

int main(void) {
  int32_t hist = -1, slots[16], ids[16];
  lf_status st = lf_cache_frame_slots(LF_CACHE_ROLLING, 9, 0, 3, 4, &hist, slots, ids);
  if (st != LF_OK) return 10;
  printf("hist %d\n", hist);
  printf("slots");
  for (int i = 0; i < hist + 3; ++i) printf(" %d", slots[i]);
  printf("\nids");
  for (int i = 0; i < hist + 3; ++i) printf(" %d", ids[i]);
  printf("\n");

  double sigma[7], spars[7], beta = 0.0;
  uint8_t dense[7];
  int32_t hf[7], kf[7], kb[7];
  for (int i = 0; i < 7; ++i) {
    sigma[i] = 0.1 + 0.9 * i / 6.0;
    dense[i] = (uint8_t)(i == 0);
    hf[i] = 3 * i;
  }
  st = lf_chunk_budget(7, sigma, NULL, dense, 0.9, 0.8, hf, NULL, 25, 3, spars, &beta, kf, kb);
  if (st != LF_OK) return 11;
  printf("beta %.12f\n", beta);

  st = lf_block_sparse_attn(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 1.0f, NULL, NULL, NULL);
  printf("null_geometry %s\n", lf_status_str(st));
  return 0;
}
"""


def test_c_program_against_lf_h(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.dirname(lf.LIB_PATH)
    if not os.path.exists(lf.LIB_PATH):
        pytest.skip("liblf.so not built")
    src = tmp_path / "use_lf.c"
    src.write_text(SRC)
    exe = tmp_path / "use_lf"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-o", str(exe), lib_dir + "/liblf.so", "-Wl,-rpath," + lib_dir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    assert out[0] == "hist 6"
    assert out[1].split()[1:] == [str(a % 9) for a in range(6, 15)]
    assert out[2].split()[1:] == [str(a) for a in range(6, 15)]
    beta = float(out[3].split()[1])
    want = (0.9 - 0.8) * 6 / sum(1.0 / math.sqrt(0.1 + 0.9 * i / 6.0) for i in range(1, 7))
    assert abs(beta - want) < 1e-12 and abs(beta - 0.073087) < 5e-7
    assert out[4] == "null_geometry LF_ERR_NULL"
