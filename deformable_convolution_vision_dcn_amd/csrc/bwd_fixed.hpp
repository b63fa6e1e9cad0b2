// bwd_fixed.hpp -- pieces shared by the LDS-windowed backward kernels: the
// fixed-point channel pairs of the grad window and the lane-constant slices
// that stage a window and flush it.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace dcn {

// Two neighbouring channels' fixed-point terms added by one 64-bit LDS
// integer add (ds_add_u64) at LDS byte address `addr`.  The pair is the
// 64-bit integer hi * 2^32 + lo (lo sign-extended into the high word), so a
// sum of such terms is (sum hi) * 2^32 + sum lo exactly, and as long as
// |sum lo| < 2^31 both sums come back from it (see pair_sums).
__device__ __forceinline__ void lds_add_pair(uint32_t addr, int lo, int hi) {
  typedef __attribute__((address_space(3))) uint64_t L;
  const uint64_t v = ((uint64_t)(uint32_t)(hi + (lo >> 31)) << 32) | (uint32_t)lo;
  __hip_atomic_fetch_add((L *)(size_t)addr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int2 pair_sums(uint64_t v) {
  const int lo = (int)(uint32_t)v;
  const int hi = (int)((int64_t)(v - (uint64_t)(int64_t)lo) >> 32);
  return make_int2(lo, hi);
}

// Lane-constant slices of a SW x SH window for WP lane groups: main slice u
// holds rows [u RPS, u RPS + RPS) of columns [0, CW) (CW divides WP, so
// every group has a pixel in every main slice), remainder slice rho the
// pixels rho WP + group of the rows below (columns [0, CW)) and then of the
// columns right of that block.  A group keeps its column in every main
// slice, so per item a main slice costs one add.
constexpr int slice_width(int sw, int wp) {
  int c = sw < 32 ? sw : 32;
  while (c > 1 && wp % c != 0) --c;
  return c;
}
template <int SW, int SH, int WP>
struct Slices {
  static constexpr int CW = slice_width(SW, WP);
  static constexpr int RPS = WP / CW;
  static constexpr int NM = SH / RPS;
  static constexpr int REM_A = (SH - NM * RPS) * CW, REM_B = (SW - CW) * SH;
  static constexpr int NR = (REM_A + REM_B + WP - 1) / WP;
  static constexpr int N = NM + NR;
  static_assert(RPS >= 1 && NM >= 1, "slice geometry");
  // Window pixel (y, x) of remainder slice rho for lane group g; false if
  // the slice has no pixel for it.  (rho is a constant once the slice loop
  // is unrolled, so the divisions are by constants.)
  __device__ static __forceinline__ bool rem(int rho, uint32_t g, uint32_t &y, uint32_t &x) {
    const uint32_t rs = (uint32_t)(rho * WP) + g;
    if (rs < (uint32_t)REM_A) {
      y = (uint32_t)(NM * RPS) + rs / (uint32_t)CW;
      x = rs % (uint32_t)CW;
      return true;
    }
    if constexpr (SW > CW) {
      const uint32_t r = rs - (uint32_t)REM_A;
      y = r / (uint32_t)(SW - CW);
      x = (uint32_t)CW + r % (uint32_t)(SW - CW);
      return rs < (uint32_t)(REM_A + REM_B);
    }
    y = x = 0;
    return false;
  }
};

}  // namespace dcn
