"""Host-side arithmetic of the library that needs no GPU: the multiply-high
division used to decode prefill work items (magic numbers computed by the
library's own host code, compiled here with hipcc for the host only)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_kv_store_amd", "csrc")

PROG = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include "kvs_internal.hpp"
// device form: q = (mulhi(n, m) + n) >> l, for n < 2^31
static uint32_t q_of(uint32_t n, uint32_t m, uint32_t l) {
  const uint32_t hi = (uint32_t)(((uint64_t)n * m) >> 32);
  return (hi + n) >> l;
}
int main() {
  std::mt19937_64 rng(12345);
  long bad = 0, checked = 0;
  auto check = [&](uint32_t d, uint32_t n) {
    uint32_t m, l;
    kvs::fast_div_magic(d, &m, &l);
    ++checked;
    if (q_of(n, m, l) != n / d) {
      if (bad < 5) std::printf("mismatch d=%u n=%u got=%u want=%u\n", d, n, q_of(n, m, l), n / d);
      ++bad;
    }
  };
  const uint32_t nmax = 0x7fffffffu;
  for (uint32_t d = 1; d <= 4100; ++d) {
    for (uint32_t k = 0; k < 64; ++k) check(d, k);
    for (uint32_t k = 0; k < 64; ++k) { const uint64_t x = (uint64_t)d * (k + 1); if (x <= nmax) { check(d, (uint32_t)x); check(d, (uint32_t)x - 1); } }
    check(d, nmax); check(d, nmax - 1);
    for (int k = 0; k < 200; ++k) check(d, (uint32_t)(rng() % (nmax + 1ull)));
  }
  for (int k = 0; k < 200000; ++k) {
    const uint32_t d = 1 + (uint32_t)(rng() % nmax);
    check(d, (uint32_t)(rng() % (nmax + 1ull)));
    const uint64_t mult = (uint64_t)d * (1 + rng() % 8);
    if (mult <= nmax) { check(d, (uint32_t)mult); check(d, (uint32_t)mult - 1); }
  }
  for (uint32_t s = 0; s < 31; ++s) { check(1u << s, nmax); check((1u << s) + 1, nmax); check((1u << s) - 1 ? (1u << s) - 1 : 1, nmax); }
  std::printf("checked %ld bad %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_fast_division_magic(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    src = tmp_path / "fastdiv.cpp"
    src.write_text(PROG)
    exe = tmp_path / "fastdiv"
    subprocess.run([hipcc, "-O2", "-x", "hip", "--offload-arch=gfx950", "-I" + CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "bad 0" in r.stdout
