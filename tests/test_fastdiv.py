"""The kernels' division by a launch-time divisor (csrc/fastdiv.hpp) against the C++ `/`
operator, on the CPU: the header is compiled with g++ (its device qualifiers defined away)
and checked on every divisor up to 2^16 and on the edges of the 31-bit range."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_attention_qk_amd", "csrc")

PROGRAM = r"""
#include <stdio.h>
#include <stdint.h>
#include "fastdiv.hpp"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd31() {  // xorshift64*, top 31 bits
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 33);
}

static int check(uint32_t d, uint32_t n, const attn::FastDiv& f) {
  if (f.div(n) != n / d || f.mod(n) != n % d) {
    printf("FAIL d=%u n=%u got %u want %u\n", d, n, f.div(n), n / d);
    return 1;
  }
  return 0;
}

int main() {
  const uint32_t top = 0x7fffffffu;
  uint32_t big[] = {top, top - 1, 1u << 30, (1u << 30) + 1, (1u << 30) - 1, 3u << 29,
                    1000000007u, 65537u * 3u, 123456789u};
  int bad = 0;
  for (uint32_t d = 1; d <= (1u << 16) && !bad; ++d) {
    const attn::FastDiv f = attn::make_fastdiv(d);
    for (uint32_t n = 0; n < 3 * d + 70 && n < 4096; ++n) bad |= check(d, n, f);
    for (uint32_t n = 3 * d - 70; d > 1400 && n < 3 * d + 70; ++n) bad |= check(d, n, f);
    for (uint32_t k = 1; k < 64; ++k) {
      const uint64_t m = (uint64_t)(top / d / 64) * k * 64 / 64 * d;  // multiples of d
      for (int e = -1; e <= 1; ++e) {
        const uint64_t n = m + e;
        if (n <= top) bad |= check(d, (uint32_t)n, f);
      }
    }
    for (int i = 0; i < 64; ++i) bad |= check(d, rnd31(), f);
    bad |= check(d, top, f) | check(d, top - 1, f);
  }
  for (uint32_t d : big) {
    const attn::FastDiv f = attn::make_fastdiv(d);
    for (int i = 0; i < 200000 && !bad; ++i) bad |= check(d, rnd31(), f);
    uint32_t edges[] = {0, 1, d - 1, d, d + 1 <= top ? d + 1 : d, top, top - 1, top / 2};
    for (uint32_t n : edges) if (n <= top) bad |= check(d, n, f);
  }
  {
    const attn::FastDiv f = attn::make_fastdiv(1u << 31);  // largest divisor
    for (int i = 0; i < 1000; ++i) bad |= check(1u << 31, rnd31(), f);
  }
  printf(bad ? "failed\n" : "ok\n");
  return bad;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "fastdiv_check.cpp"
    exe = tmp_path / "fastdiv_check"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-O2", "-std=c++17", "-D__host__=", "-D__device__=",
                    "-D__forceinline__=inline", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:]
