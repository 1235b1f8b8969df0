"""The geometry header compiled for the host with g++: the per-tile interval
derivation the wide kernels use (row_interval_of_block, from a row's block)
equals row_interval, exhaustively on small shapes, in both modes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_lm_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include "geometry.h"
using namespace bd;
int main() {
  long checked = 0;
  for (int n = 1; n <= 70; ++n)
    for (int b = 1; b <= n + 3; ++b)
      for (int mode = 0; mode < 2; ++mode) {
        const Geom g{n, mode == MODE_CAUSAL ? 1 : b};
        for (int qh = 0; qh < 2; ++qh)
          for (int kh = 0; kh < 2; ++kh)
            for (int p = 0; p < n + 40; ++p) {  // rows past the half too
              int l0, h0, l1, h1;
              row_interval(g, qh, kh, p, l0, h0);
              row_interval_of_block(qh, kh, g.bstart(p), g.bend(p), l1, h1);
              if (l0 != l1 || h0 != h1) {
                printf("mismatch n=%d b=%d mode=%d qh=%d kh=%d p=%d: [%d,%d) vs [%d,%d)\n",
                       n, b, mode, qh, kh, p, l0, h0, l1, h1);
                return 1;
              }
              ++checked;
            }
      }
  printf("ok %ld\n", checked);
  return 0;
}
"""


def test_row_interval_of_block_equals_row_interval(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    src = tmp_path / "check.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "check"
    # the header's device qualifiers become plain inline functions on the host
    subprocess.run([gxx, "-std=c++17", "-O1", "-D__HIPCC__", "-D__host__=", "-D__device__=",
                    "-D__forceinline__=inline", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout
    assert r.stdout.startswith("ok")
