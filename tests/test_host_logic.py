"""Host-compilable index helpers of the kernels (index_math.hpp), built with
g++ and checked exhaustively on edge values and randomly elsewhere."""
import pathlib
import subprocess

ROOT = pathlib.Path(__file__).resolve().parents[1]
CSRC = ROOT / "deformable_convolution_vision_dcn_amd" / "csrc"

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>
#include "index_math.hpp"
int main() {
  using namespace dcn;
  std::mt19937_64 rng(7);
  long bad = 0, checked = 0;
  std::vector<uint32_t> divisors;
  for (uint32_t d = 1; d <= 4096; ++d) divisors.push_back(d);
  for (int e = 12; e < 31; ++e) {
    uint32_t p = 1u << e;
    divisors.push_back(p - 1); divisors.push_back(p); divisors.push_back(p + 1);
  }
  divisors.push_back(0x7fffffffu);
  for (int i = 0; i < 2000; ++i) divisors.push_back(1 + (uint32_t)(rng() % 0x7fffffffu));
  for (uint32_t d : divisors) {
    FastDiv f = make_fast_div(d);
    std::vector<uint32_t> ns = {0, 1, d - 1, d, d + 1, 2 * d - 1, 0x7fffffffu, 0x7ffffffeu};
    for (int i = 0; i < 200; ++i) ns.push_back((uint32_t)(rng() % 0x80000000u));
    for (uint32_t k = 1; k < 50; ++k) { uint64_t m = (uint64_t)k * d; if (m < 0x80000000u) { ns.push_back((uint32_t)m); ns.push_back((uint32_t)m - 1); } }
    for (uint32_t n : ns) {
      if (n >= 0x80000000u) continue;
      ++checked;
      if (fast_div(n, f) != n / d) { if (bad < 5) printf("bad n=%u d=%u\n", n, d); ++bad; }
    }
  }
  // xcd_block is a bijection of [0, nb) with contiguous ranges per XCD
  for (uint32_t nb = 1; nb <= 3000; nb += (nb < 100 ? 1 : 37)) {
    std::vector<int> seen(nb, 0);
    for (uint32_t b = 0; b < nb; ++b) {
      uint32_t l = xcd_block(b, nb);
      if (l >= nb || seen[l]++) { printf("xcd not bijective nb=%u\n", nb); return 1; }
      if (b >= 8 && xcd_block(b, nb) != xcd_block(b - 8, nb) + 1) { printf("xcd not contiguous nb=%u\n", nb); return 1; }
    }
  }
  // xcd_walk: every item exactly once, each XCD's items one contiguous range
  for (uint32_t nb = 1; nb <= 1100; nb += (nb < 40 ? 1 : 53)) {
    for (uint32_t items : {0u, 1u, 7u, 8u, 9u, nb - 1, nb, nb + 1, 3 * nb + 5, 11520u, 100003u}) {
      std::vector<int> seen(items, 0);
      std::vector<uint32_t> lo(8, 0xffffffffu), hi(8, 0), cnt(8, 0);
      for (uint32_t b = 0; b < nb; ++b) {
        XcdWalk w = xcd_walk(b, nb, items);
        if (w.stride == 0) { printf("zero stride nb=%u\n", nb); return 1; }
        for (uint32_t it = w.first; it < w.end; it += w.stride) {
          if (it >= items || seen[it]++) { printf("walk not a partition nb=%u items=%u\n", nb, items); return 1; }
          uint32_t x = b % 8;
          lo[x] = it < lo[x] ? it : lo[x]; hi[x] = it > hi[x] ? it : hi[x]; ++cnt[x];
        }
      }
      for (uint32_t i = 0; i < items; ++i) if (!seen[i]) { printf("item %u missed nb=%u\n", i, nb); return 1; }
      for (int x = 0; x < 8; ++x) if (cnt[x] && hi[x] - lo[x] + 1 != cnt[x]) { printf("xcd range gap nb=%u\n", nb); return 1; }
    }
  }
  printf("checked %ld bad %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_index_math(tmp_path):
    src = tmp_path / "t.cpp"
    exe = tmp_path / "t"
    src.write_text(PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O2", "-fsanitize=address,undefined",
                    f"-I{CSRC}", str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bad 0" in r.stdout
