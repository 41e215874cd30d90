"""The launch-constant division of the kernels' job mapping (``make_fastdiv`` /
``fast_div`` in ``csrc/common.h``, host and device code alike), compiled for the
host and checked against integer division: every divisor up to 4096 and a
geometric sweep to 2^31 - 1, numerators 0 .. 4999, multiples of the divisor and
their predecessors, the top of the range and random draws."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_gqa_causal_amd", "csrc")

SRC = r"""
#include "common.h"
#include <cstdio>
#include <random>
using namespace gqa;
static long bad = 0, checked = 0;
static void chk(const FastDiv& f, int n) {
  ++checked;
  if (fast_div(n, f) != n / (int)f.d && bad++ < 5) printf("d=%u n=%d got %d\n", f.d, n, fast_div(n, f));
}
int main() {
  std::mt19937 rng(7);
  for (uint64_t d = 1; d <= 0x7fffffffu; d = d < 4096 ? d + 1 : d * 5 / 4 + 1) {
    const FastDiv f = make_fastdiv((uint32_t)d);
    for (int n = 0; n < 5000; ++n) chk(f, n);
    for (int k = 0; k < 500; ++k) chk(f, (int)(rng() & 0x7fffffff));
    for (int n = 0x7fffffff; n > 0x7fffffff - 500; --n) chk(f, n);
    for (uint64_t m = 1; m < 300 && m * d <= 0x7fffffffu; ++m) { chk(f, (int)(m * d)); chk(f, (int)(m * d - 1)); }
  }
  printf("checked %ld bad %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_fast_div_matches_integer_division(tmp_path):
    hipcc = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    src = tmp_path / "fast_div_check.cpp"
    src.write_text(SRC)
    exe = tmp_path / "fast_div_check"
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC, str(src), "-o",
                        str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bad 0" in r.stdout
