// dcn_device.hpp -- device-side building blocks shared by the forward and
// backward kernels of the DCN core (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn_launch.hpp"

namespace dcn {

// Largest ratio between a tile's fixed-point bound B (the sum over its
// pixel-groups of sum_k |m_k| * max_c |gy_c|) and its smallest nonzero
// per-pixel-group term for which the tiled backward kernels accumulate
// grad_input in fixed point; a wider spread takes fp32 atomics.
constexpr float kFixedSpread = 4096.f;

// ---------------------------------------------------------------- raw buffers
// A raw buffer resource (stride 0, num_records in bytes).  Loads whose byte
// offset lies beyond num_records return 0 and stores/atomics there are
// dropped by the hardware, which is how corners outside the feature map are
// read as zero without a branch: their offset is set to kOutOfRange.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw-buffer format word

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Load NW 32-bit words (NW in {1, 2, 4, 8, 16}) at byte offset voff.
template <int NW>
__device__ __forceinline__ void buffer_load_words(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
  } else if constexpr (NW == 2) {
    auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
    w[0] = v[0];
    w[1] = v[1];
  } else {
    static_assert(NW % 4 == 0, "word count");
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 16u * q), 0, 0);
      w[4 * q + 0] = v[0];
      w[4 * q + 1] = v[1];
      w[4 * q + 2] = v[2];
      w[4 * q + 3] = v[3];
    }
  }
}

// Store NW 32-bit words (NW in {1, 2, 4}) at byte offset voff; offsets beyond
// num_records are dropped by the hardware.
// An empty asm that claims to modify its operands: the values must exist in
// registers at this point of the program.  Used to keep a chain of FMAs next
// to the loads that feed it: left alone, the compiler sinks pure arithmetic
// to its last use and keeps every loaded operand live until then.
template <int N>
__device__ __forceinline__ void pin_values(float (&v)[N]) {
  static_assert(N == 4 || N == 8, "four or eight values");
  if constexpr (N == 4) {
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
  } else {
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                 "+v"(v[7]));
  }
}

// AUX: the cache-policy operand of the buffer instruction (0 = default).
constexpr int kNonTemporal = 2;  // the nt bit: streamed, evicted first
template <int NW, int AUX>
__device__ __forceinline__ void buffer_store_words_aux(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                       const uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], r, (int)voff, 0, AUX);
  } else if constexpr (NW == 2) {
    typedef uint32_t v2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(v2{w[0], w[1]}, r, (int)voff, 0, AUX);
  } else {
    static_assert(NW == 4, "word count");
    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(v4{w[0], w[1], w[2], w[3]}, r, (int)voff, 0, AUX);
  }
}

template <int NW>
__device__ __forceinline__ void buffer_store_words(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                   const uint32_t (&w)[NW]) {
  buffer_store_words_aux<NW, 0>(r, voff, w);
}

// ---------------------------------------------------------------- I/O types
template <int DT> struct Io;
template <> struct Io<DCN_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerWord = 1;
  __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w); }
  __device__ static __forceinline__ float one(const void *p, int64_t i) {
    return static_cast<const float *>(p)[i];
  }
};
template <> struct Io<DCN_F16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerWord = 2;
  __device__ static __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  __device__ static __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  __device__ static __forceinline__ float one(const void *p, int64_t i) {
    return (float)static_cast<const _Float16 *>(p)[i];
  }
  __device__ static __forceinline__ uint32_t pack(float a, float b) {
    uint32_t l = __builtin_bit_cast(uint16_t, (_Float16)a);
    uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)b);
    return l | (h << 16);
  }
};
template <> struct Io<DCN_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerWord = 2;
  __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static __forceinline__ float one(const void *p, int64_t i) {
    return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
  }
  __device__ static __forceinline__ uint32_t pack(float a, float b) {
    uint32_t l = __builtin_bit_cast(uint16_t, (__bf16)a);
    uint32_t h = __builtin_bit_cast(uint16_t, (__bf16)b);
    return l | (h << 16);
  }
};

// Widen NW words into NW * kPerWord floats.
template <int DT, int NW>
__device__ __forceinline__ void unpack(const uint32_t (&w)[NW], float (&v)[NW * Io<DT>::kPerWord]) {
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if constexpr (DT == DCN_F32) {
      v[i] = Io<DT>::lo(w[i]);
    } else {
      v[2 * i] = Io<DT>::lo(w[i]);
      v[2 * i + 1] = Io<DT>::hi(w[i]);
    }
  }
}

// Narrow NV floats into NV / kPerWord words (round to nearest even).
template <int DT, int NV>
__device__ __forceinline__ void pack_words(const float (&v)[NV], uint32_t (&w)[NV / Io<DT>::kPerWord]) {
#pragma unroll
  for (int i = 0; i < NV / Io<DT>::kPerWord; ++i) {
    if constexpr (DT == DCN_F32) {
      w[i] = __float_as_uint(v[i]);
    } else {
      w[i] = Io<DT>::pack(v[2 * i], v[2 * i + 1]);
    }
  }
}

// Store NW words to a 16-byte-aligned global address (vector stores).
template <int NW>
__device__ __forceinline__ void store_words(void *dst, const uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    *static_cast<uint32_t *>(dst) = w[0];
  } else if constexpr (NW == 2) {
    *static_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
  } else {
    static_assert(NW % 4 == 0, "word count");
#pragma unroll
    for (int q = 0; q < NW / 4; ++q)
      static_cast<uint4 *>(dst)[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
  }
}

// Copy nbytes (a multiple of 2) from 16-byte-aligned global memory into LDS,
// with the whole block cooperating.  16-byte vector copies for the bulk,
// 2-byte copies for the tail.
__device__ __forceinline__ void stage_to_lds(void *lds, const void *src, uint32_t nbytes) {
  const uint32_t n16 = nbytes / 16;
  const uint4 *s4 = static_cast<const uint4 *>(src);
  uint4 *d4 = static_cast<uint4 *>(lds);
  for (uint32_t i = threadIdx.x; i < n16; i += blockDim.x) d4[i] = s4[i];
  const uint32_t done = n16 * 16;
  const uint16_t *s2 = static_cast<const uint16_t *>(src);
  uint16_t *d2 = static_cast<uint16_t *>(lds);
  for (uint32_t i = done / 2 + threadIdx.x; i < nbytes / 2; i += blockDim.x) d2[i] = s2[i];
}

// Row loads of one pixel-group's offsets and mask values (wide loads at the
// rows' 4-byte alignment).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// The K (x, y) offset pairs of pixel-group pg as 2K fp32 values, for the 9
// points of a 3x3 kernel or the 8 left without its centre.
template <int DT, int K>
__device__ __forceinline__ void load_offsets(const void *base, uint32_t pg, float (&o)[2 * K]) {
  static_assert(K == 9 || K == 8, "3x3 rows");
  if constexpr (DT == DCN_F32) {
    const uint32_t *src = static_cast<const uint32_t *>(base) + (uint64_t)pg * (2 * K);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(src + 4 * q);
      o[4 * q] = __uint_as_float(v[0]);
      o[4 * q + 1] = __uint_as_float(v[1]);
      o[4 * q + 2] = __uint_as_float(v[2]);
      o[4 * q + 3] = __uint_as_float(v[3]);
    }
    if constexpr (K == 9) {
      const u32x2_a4 v = *reinterpret_cast<const u32x2_a4 *>(src + 16);
      o[16] = __uint_as_float(v[0]);
      o[17] = __uint_as_float(v[1]);
    }
  } else {
    const uint32_t *src = static_cast<const uint32_t *>(base) + (uint64_t)pg * K;
    uint32_t w[K];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(src + 4 * q);
      w[4 * q] = v[0];
      w[4 * q + 1] = v[1];
      w[4 * q + 2] = v[2];
      w[4 * q + 3] = v[3];
    }
    if constexpr (K == 9) w[8] = src[8];
#pragma unroll
    for (int q = 0; q < K; ++q) {
      o[2 * q] = Io<DT>::lo(w[q]);
      o[2 * q + 1] = Io<DT>::hi(w[q]);
    }
  }
}

// The K mask values of pixel-group pg as fp32 (K = 9 or 8 as above).
template <int DT, int K>
__device__ __forceinline__ void load_mask(const void *base, uint32_t pg, float (&m)[K]) {
  static_assert(K == 9 || K == 8, "3x3 rows");
  if constexpr (DT == DCN_F32) {
    const uint32_t *src = static_cast<const uint32_t *>(base) + (uint64_t)pg * K;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(src + 4 * q);
      m[4 * q] = __uint_as_float(v[0]);
      m[4 * q + 1] = __uint_as_float(v[1]);
      m[4 * q + 2] = __uint_as_float(v[2]);
      m[4 * q + 3] = __uint_as_float(v[3]);
    }
    if constexpr (K == 9) m[8] = __uint_as_float(src[8]);
  } else if constexpr (K == 8) {  // 16-byte rows: one aligned 16-byte load
    const uint32_t *src = static_cast<const uint32_t *>(base) + (uint64_t)pg * 4;
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(src);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m[2 * q] = Io<DT>::lo(v[q]);
      m[2 * q + 1] = Io<DT>::hi(v[q]);
    }
  } else {
    const uint16_t *src = static_cast<const uint16_t *>(base) + (uint64_t)pg * K;
#pragma unroll
    for (int q = 0; q < K; ++q) m[q] = Io<DT>::lo((uint32_t)src[q]);
  }
}

// Offsets and mask values of one pixel-group of a 3x3 problem, kept as the
// raw words the loads return (decoded where used, so that issuing the loads
// does not wait for them).  fp32: 18 offset words (x, y per point) and 9
// mask words.  16-bit: 9 offset words ((x, y) per point) and 5 words that
// cover the 18-byte mask row.  Every load is a buffer load of at most 16
// bytes at a 4-byte-aligned offset inside the tensor: the 16-bit mask row of
// an odd pixel-group starts 2 bytes into a word, so its words are read from
// 2 bytes before the row (the previous row's last value, ignored) to the row
// end, and an even row's last value comes from a 2-byte load.
template <int DT, int K = 9>
struct RowWords {
  static_assert(K == 9 || K == 8, "3x3 rows");
  static constexpr int kOff = DT == DCN_F32 ? 2 * K : K;
  static constexpr int kMask = DT == DCN_F32 ? K : (K == 9 ? 5 : 4);
  uint32_t o[kOff], m[kMask];
};

template <int DT, int K = 9>
__device__ __forceinline__ void load_row_words(__amdgpu_buffer_rsrc_t roff, __amdgpu_buffer_rsrc_t rmask,
                                               uint32_t pg, RowWords<DT, K> &r) {
  if constexpr (K == 8) {
    // Rows of 8 points are 16-byte aligned in every dtype: whole b128 loads.
    constexpr int NO = RowWords<DT, K>::kOff / 4, NM = RowWords<DT, K>::kMask / 4;
    const uint32_t o = pg * (uint32_t)(16 * NO), m = pg * (uint32_t)(16 * NM);
#pragma unroll
    for (int q = 0; q < NO; ++q) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(roff, (int)(o + 16 * q), 0, 0);
      r.o[4 * q] = v[0];
      r.o[4 * q + 1] = v[1];
      r.o[4 * q + 2] = v[2];
      r.o[4 * q + 3] = v[3];
    }
#pragma unroll
    for (int q = 0; q < NM; ++q) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rmask, (int)(m + 16 * q), 0, 0);
      r.m[4 * q] = v[0];
      r.m[4 * q + 1] = v[1];
      r.m[4 * q + 2] = v[2];
      r.m[4 * q + 3] = v[3];
    }
  } else if constexpr (DT == DCN_F32) {
    const uint32_t o = pg * 72u, m = pg * 36u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(roff, (int)(o + 16 * q), 0, 0);
      r.o[4 * q] = v[0];
      r.o[4 * q + 1] = v[1];
      r.o[4 * q + 2] = v[2];
      r.o[4 * q + 3] = v[3];
    }
    const auto v8 = __builtin_amdgcn_raw_buffer_load_b64(roff, (int)(o + 64), 0, 0);
    r.o[16] = v8[0];
    r.o[17] = v8[1];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rmask, (int)(m + 16 * q), 0, 0);
      r.m[4 * q] = v[0];
      r.m[4 * q + 1] = v[1];
      r.m[4 * q + 2] = v[2];
      r.m[4 * q + 3] = v[3];
    }
    r.m[8] = __builtin_amdgcn_raw_buffer_load_b32(rmask, (int)(m + 32), 0, 0);
  } else {
    const uint32_t o = pg * 36u, m = pg * 18u, a = m & ~3u;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(roff, (int)(o + 16 * q), 0, 0);
      r.o[4 * q] = v[0];
      r.o[4 * q + 1] = v[1];
      r.o[4 * q + 2] = v[2];
      r.o[4 * q + 3] = v[3];
    }
    r.o[8] = __builtin_amdgcn_raw_buffer_load_b32(roff, (int)(o + 32), 0, 0);
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rmask, (int)a, 0, 0);
    r.m[0] = v[0];
    r.m[1] = v[1];
    r.m[2] = v[2];
    r.m[3] = v[3];
    const bool odd = (m & 2u) != 0;
    const uint32_t w4a = __builtin_amdgcn_raw_buffer_load_b32(rmask, odd ? (int)(a + 16) : (int)kOutOfRange, 0, 0);
    const uint32_t w4b = __builtin_amdgcn_raw_buffer_load_b16(rmask, odd ? (int)kOutOfRange : (int)(a + 16), 0, 0);
    r.m[4] = w4a | w4b;
  }
}

// The K mask values of load_row_words as fp32.
template <int DT, int K = 9>
__device__ __forceinline__ void decode_mask_words(uint32_t pg, const RowWords<DT, K> &r, float (&msk)[K]) {
  if constexpr (DT == DCN_F32) {
#pragma unroll
    for (int q = 0; q < K; ++q) msk[q] = __uint_as_float(r.m[q]);
  } else if constexpr (K == 8) {  // aligned rows: two values per word
#pragma unroll
    for (int q = 0; q < 8; ++q) msk[q] = (q & 1) ? Io<DT>::hi(r.m[q / 2]) : Io<DT>::lo(r.m[q / 2]);
  } else {
    const uint32_t sh = (pg * 18u) & 2u ? 16u : 0u;  // odd pg: the row starts at a half word
    uint32_t w[5];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = __builtin_amdgcn_alignbit(r.m[q + 1], r.m[q], sh);
    w[4] = r.m[4] >> sh;
#pragma unroll
    for (int q = 0; q < 9; ++q) msk[q] = (q & 1) ? Io<DT>::hi(w[q / 2]) : Io<DT>::lo(w[q / 2]);
  }
}

// Offset (x, y) of point k of load_row_words as fp32.
template <int DT, int K = 9>
__device__ __forceinline__ void offset_words_xy(const RowWords<DT, K> &r, int k, float &x, float &y) {
  if constexpr (DT == DCN_F32) {
    x = __uint_as_float(r.o[2 * k]);
    y = __uint_as_float(r.o[2 * k + 1]);
  } else {
    x = Io<DT>::lo(r.o[k]);
    y = Io<DT>::hi(r.o[k]);
  }
}

// The 2K offsets (x, y per point) and K mask values of load_row_words as fp32.
template <int DT, int K = 9>
__device__ __forceinline__ void decode_row_words(uint32_t pg, const RowWords<DT, K> &r, float (&off)[2 * K],
                                                 float (&msk)[K]) {
  if constexpr (DT == DCN_F32) {
#pragma unroll
    for (int q = 0; q < 2 * K; ++q) off[q] = __uint_as_float(r.o[q]);
#pragma unroll
    for (int q = 0; q < K; ++q) msk[q] = __uint_as_float(r.m[q]);
  } else {
#pragma unroll
    for (int q = 0; q < K; ++q) {
      off[2 * q] = Io<DT>::lo(r.o[q]);
      off[2 * q + 1] = Io<DT>::hi(r.o[q]);
    }
    if constexpr (K == 8) {  // aligned rows: two values per word
#pragma unroll
      for (int q = 0; q < 8; ++q) msk[q] = (q & 1) ? Io<DT>::hi(r.m[q / 2]) : Io<DT>::lo(r.m[q / 2]);
    } else {
      const uint32_t sh = (pg * 18u) & 2u ? 16u : 0u;  // odd pg: the row starts at a half word
      uint32_t w[5];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = __builtin_amdgcn_alignbit(r.m[q + 1], r.m[q], sh);
      w[4] = r.m[4] >> sh;
#pragma unroll
      for (int q = 0; q < 9; ++q) msk[q] = (q & 1) ? Io<DT>::hi(w[q / 2]) : Io<DT>::lo(w[q / 2]);
    }
  }
}

}  // namespace dcn
