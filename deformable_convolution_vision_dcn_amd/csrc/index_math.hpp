// index_math.hpp -- integer index helpers used by the kernels, written so
// that host-only tests can compile them with a plain C++ compiler.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DCN_HD __host__ __device__
#else
#define DCN_HD
#endif

namespace dcn {

// Division by a run-time invariant divisor (Granlund & Montgomery, "Division
// by invariant integers using multiplication", PLDI 1994).  For
// 1 <= d < 2^31 and dividends n < 2^31:
//   n / d == (mulhi32(n, mul) + n) >> shift
// with shift = ceil(log2 d) and mul = floor(2^32 * (2^shift - d) / d) + 1.
struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

inline FastDiv make_fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{static_cast<uint32_t>(m), l};
}

DCN_HD inline uint32_t fast_div(uint32_t n, FastDiv f) {
  const uint32_t hi = static_cast<uint32_t>((uint64_t(n) * f.mul) >> 32);
  return (hi + n) >> f.shift;
}

// Blocks are handed to the 8 XCDs of the chip round-robin (block b runs on
// XCD b % 8).  This bijection of [0, nb) gives each XCD one contiguous run of
// logical blocks, so neighbouring output pixels -- whose sampling windows
// overlap -- are processed by one XCD and meet in its L2.
DCN_HD inline uint32_t xcd_block(uint32_t b, uint32_t nb) {
  constexpr uint32_t kXcd = 8;
  const uint32_t x = b % kXcd, i = b / kXcd;
  const uint32_t per = nb / kXcd, rem = nb % kXcd;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

// Work split of a persistent launch of nb blocks over `items` work items:
// XCD x takes one contiguous range of items, sized in proportion to the
// blocks it runs, and its blocks walk that range in step (first = start +
// local block index, stride = blocks on the XCD).  Work items that are close
// in index -- neighbouring tiles, whose input windows overlap -- are then
// processed by one XCD close in time and share its L2, instead of being
// dealt round-robin to all eight.
struct XcdWalk {
  uint32_t first, stride, end;
};

DCN_HD inline XcdWalk xcd_walk(uint32_t b, uint32_t nb, uint32_t items) {
  constexpr uint32_t kXcd = 8;
  const uint32_t x = b % kXcd, i = b / kXcd;
  const uint32_t per = nb / kXcd, rem = nb % kXcd;
  const uint32_t per_x = per + (x < rem ? 1u : 0u);
  const uint32_t lo = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  const uint32_t start = static_cast<uint32_t>(uint64_t(items) * lo / nb);
  const uint32_t end = static_cast<uint32_t>(uint64_t(items) * (lo + per_x) / nb);
  return XcdWalk{start + i, per_x, end};
}

}  // namespace dcn
