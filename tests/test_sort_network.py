"""Host check of the 8-key comparator network used by the 8:16 selection
(CPU only): compiled with g++ from the library's own header, it must sort every
0/1 input (the 0-1 principle then covers all inputs), and the half-cleaner over
two sorted halves must yield the 8th-largest of 16 unique keys."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR_DIR = os.path.join(ROOT, "activation_sparsity_fp4_amd", "csrc")

PROGRAM = r"""
#include <algorithm>
#include <cstdio>
#include <cstdint>
#include <random>
#include "sort_network.h"
using namespace sharq;
static void sort8(uint32_t* a) {
  for (int c = 0; c < kSort8Size; ++c) {
    int i = kSort8[c][0], j = kSort8[c][1];
    uint32_t hi = std::max(a[i], a[j]), lo = std::min(a[i], a[j]);
    a[i] = hi; a[j] = lo;
  }
}
int main() {
  for (int bits = 0; bits < 256; ++bits) {
    uint32_t a[8], s[8];
    for (int i = 0; i < 8; ++i) a[i] = s[i] = (bits >> i) & 1;
    sort8(a);
    std::sort(s, s + 8, [](uint32_t x, uint32_t y) { return x > y; });
    for (int i = 0; i < 8; ++i) if (a[i] != s[i]) { printf("FAIL01 %d\n", bits); return 1; }
  }
  std::mt19937 rng(1);
  for (int trial = 0; trial < 100000; ++trial) {
    uint32_t k[16];
    for (int i = 0; i < 16; ++i) k[i] = ((rng() % 7) << 4) | (15 - i);  // ties broken by index bits
    uint32_t lo[8], hi[8];
    for (int i = 0; i < 8; ++i) { lo[i] = k[i]; hi[i] = k[8 + i]; }
    sort8(lo); sort8(hi);
    uint32_t thr = 0xFFFFFFFFu;
    for (int i = 0; i < 8; ++i) thr = std::min(thr, std::max(lo[i], hi[7 - i]));
    uint32_t s[16];
    std::copy(k, k + 16, s);
    std::sort(s, s + 16, [](uint32_t x, uint32_t y) { return x > y; });
    if (thr != s[7]) { printf("FAILthr\n"); return 1; }
  }
  printf("OK\n");
  return 0;
}
"""


def test_sort_network_zero_one_principle_and_threshold():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.cpp")
        exe = os.path.join(d, "t")
        with open(src, "w") as f:
            f.write(PROGRAM)
        subprocess.run([gxx, "-std=c++17", "-O1", "-I", HDR_DIR, src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True)
        assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout
