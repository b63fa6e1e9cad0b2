// quad_ops.hpp -- lane-quad helpers shared by the tiled forward and backward
// kernels: DPP broadcasts within a quad of lanes (alone or as an operand of
// the instruction that consumes them), quad reductions, LDS access by
// absolute address and 24-bit integer multiplies.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace dcn {

template <int O>
__device__ __forceinline__ int qbcast(int v) {
  constexpr int ctrl = O | (O << 2) | (O << 4) | (O << 6);  // quad_perm [O,O,O,O]
  return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, false);
}
template <int O>
__device__ __forceinline__ float qbcast(float v) {
  return __int_as_float(qbcast<O>(__float_as_int(v)));
}

// acc[c] += w(lane O of the quad) * v[c]: the broadcast rides on the FMA as a
// DPP operand instead of a separate move.  The compiler does not look inside
// asm for the DPP hazard (a VALU write of w then a DPP read of it needs two
// wait states), hence the s_nop.
#define DCN_FMA4_DPP(QP)                                                              \
  asm("s_nop 1\n\t"                                                                  \
      "v_fmac_f32_dpp %0, %4, %5 " QP " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %1, %4, %6 " QP " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %2, %4, %7 " QP " row_mask:0xf bank_mask:0xf\n\t"              \
      "v_fmac_f32_dpp %3, %4, %8 " QP " row_mask:0xf bank_mask:0xf"                    \
      : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])                        \
      : "v"(w), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]))
template <int O>
__device__ __forceinline__ void fma4_bcast(float (&acc)[4], float w, const float (&v)[4]) {
  if constexpr (O == 0) DCN_FMA4_DPP("quad_perm:[0,0,0,0]");
  if constexpr (O == 1) DCN_FMA4_DPP("quad_perm:[1,1,1,1]");
  if constexpr (O == 2) DCN_FMA4_DPP("quad_perm:[2,2,2,2]");
  if constexpr (O == 3) DCN_FMA4_DPP("quad_perm:[3,3,3,3]");
}
#undef DCN_FMA4_DPP

// a(lane O of the quad) + b, the broadcast again a DPP operand.
#define DCN_ADD_DPP(QP)                                                               \
  asm("s_nop 1\n\tv_add_u32_dpp %0, %1, %2 " QP " row_mask:0xf bank_mask:0xf"         \
      : "=v"(r) : "v"(a), "v"(b))
template <int O>
__device__ __forceinline__ uint32_t add_bcast(uint32_t a, uint32_t b) {
  uint32_t r;
  if constexpr (O == 0) DCN_ADD_DPP("quad_perm:[0,0,0,0]");
  if constexpr (O == 1) DCN_ADD_DPP("quad_perm:[1,1,1,1]");
  if constexpr (O == 2) DCN_ADD_DPP("quad_perm:[2,2,2,2]");
  if constexpr (O == 3) DCN_ADD_DPP("quad_perm:[3,3,3,3]");
  return r;
}
#undef DCN_ADD_DPP

// Maximum and sum over the four lanes of a quad, one fused DPP instruction
// per butterfly step.  The maximum drops a quiet NaN operand like fmaxf.
__device__ __forceinline__ float quad_max(float v) {
  float t, r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "=&v"(t) : "v"(v));
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "=&v"(r) : "v"(t));
  return r;
}
__device__ __forceinline__ float quad_sum(float v) {
  float t, r;
  asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "=&v"(t) : "v"(v));
  asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "=&v"(r) : "v"(t));
  return r;
}

template <int NW>
__device__ __forceinline__ void lds_store(unsigned char *dst, const uint32_t (&w)[NW]) {
  if constexpr (NW == 4) {
    *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
  }
}
// Read NW words at LDS byte address `addr` (an address, not an offset from a
// generic pointer, so no base is added on the per-point path).
template <int NW>
__device__ __forceinline__ void lds_load_at(uint32_t addr, uint32_t (&w)[NW]) {
  typedef uint32_t V __attribute__((ext_vector_type(NW)));
  typedef __attribute__((address_space(3))) const V L;
  const V v = *(L *)(size_t)addr;
#pragma unroll
  for (int i = 0; i < NW; ++i) w[i] = v[i];
}

// a * b + c on the 24-bit multiplier (full rate; a, b < 2^24).
__device__ __forceinline__ uint32_t mad24(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "v"(c));
  return r;
}
__device__ __forceinline__ uint32_t mul24(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_mul_u32_u24 %0, %2, %1" : "=v"(r) : "v"(a), "s"(b));
  return r;
}


// w(lane O of the quad) * x, the broadcast a DPP operand of the multiply.
#define DCN_MUL_DPP(QP)                                                               \
  asm("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 " QP " row_mask:0xf bank_mask:0xf"         \
      : "=v"(r) : "v"(w), "v"(x))
template <int O>
__device__ __forceinline__ float mul_bcast(float w, float x) {
  float r;
  if constexpr (O == 0) DCN_MUL_DPP("quad_perm:[0,0,0,0]");
  if constexpr (O == 1) DCN_MUL_DPP("quad_perm:[1,1,1,1]");
  if constexpr (O == 2) DCN_MUL_DPP("quad_perm:[2,2,2,2]");
  if constexpr (O == 3) DCN_MUL_DPP("quad_perm:[3,3,3,3]");
  return r;
}
#undef DCN_MUL_DPP

// r[i] = w(lane O of the quad) * x[i] for four x, one hazard wait for all.
#define DCN_MUL4_DPP(QP)                                                              \
  asm("s_nop 1\n\t"                                                                  \
      "v_mul_f32_dpp %0, %4, %5 " QP " row_mask:0xf bank_mask:0xf\n\t"               \
      "v_mul_f32_dpp %1, %4, %6 " QP " row_mask:0xf bank_mask:0xf\n\t"               \
      "v_mul_f32_dpp %2, %4, %7 " QP " row_mask:0xf bank_mask:0xf\n\t"               \
      "v_mul_f32_dpp %3, %4, %8 " QP " row_mask:0xf bank_mask:0xf"                     \
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])                            \
      : "v"(w), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]))
template <int O>
__device__ __forceinline__ void mul4_bcast(float (&r)[4], float w, const float (&x)[4]) {
  if constexpr (O == 0) DCN_MUL4_DPP("quad_perm:[0,0,0,0]");
  if constexpr (O == 1) DCN_MUL4_DPP("quad_perm:[1,1,1,1]");
  if constexpr (O == 2) DCN_MUL4_DPP("quad_perm:[2,2,2,2]");
  if constexpr (O == 3) DCN_MUL4_DPP("quad_perm:[3,3,3,3]");
}
#undef DCN_MUL4_DPP

// Quad sums of four values (every lane gets all four), the swizzles DPP
// operands of the adds.  One hazard wait covers the inputs; the second step
// reads results written at least three instructions earlier.
__device__ __forceinline__ void quad_sum4(float (&v)[4]) {
  float t0, t1, t2, t3;
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %5, %5 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %6, %6 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %3, %7, %7 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
  asm("v_add_f32_dpp %0, %4, %4 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %5, %5 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %6, %6 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %3, %7, %7 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(t0), "v"(t1), "v"(t2), "v"(t3));
}

// floor(x + 0.5) as an integer in one instruction (round half up).
__device__ __forceinline__ int cvt_rpi(float x) {
  int r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

}  // namespace dcn
