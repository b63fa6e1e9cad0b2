// dcn_backward.hip -- gfx950 backward kernel of the DCNv3/DCNv4 sampling core
// (fp32), plus the fill kernel that clears grad_input before the scatter and
// the kernel that rounds an fp32 grad_input into a 16-bit one.
//
// Derivatives of the forward (wmrh.cn/news/61976, section 二 steps 2-4):
//   out_c = sum_k m_k * B_k[c],  B_k[c] = sum over the 4 corners of
//           (1-|py-yc|)(1-|px-xc|) X[yc, xc, c]  (zero outside the map)
//   grad_input  : every in-map corner receives m_k * w_corner * gy_c
//                 (scattered with fp32 atomics: many samples hit one pixel);
//   grad_offset : s * m_k * sum_c gy_c * dB_k[c]/d(px, py), stored (x, y);
//                 dB/dpy = sum_xc wx * (X[y0+1, xc] - X[y0, xc]) and likewise
//                 for px (one-sided from the right at integer coordinates);
//   grad_mask   : gm_k = sum_c gy_c * B_k[c], then through the softmax
//                 Jacobian, gl_k = m_k * (gm_k - sum_j m_j gm_j), for DCNv3.
//
// Mapping of the untiled kernel: 16 lanes per pixel-group, one channel per
// lane, so a corner gather and a corner scatter are each one 64-byte request
// per pixel-group (fp32 atomics add one value per lane: with a quad of lanes
// per pixel-group a corner took four atomic requests).  The three per-point
// channel sums are reduced over the 16 lanes with four DPP steps.  The
// grad_input scatter uses raw buffer atomics: a corner outside the map carries
// a byte offset beyond the buffer, and the hardware drops that atomic.
#include <stdlib.h>
#include <string.h>

#include "dcn_device.hpp"

namespace dcn {

namespace {

// Sum of v over the 16 lanes of a DPP row (rotations by 8 and 4 within the
// row, then the two quad permutes); every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  return v;
}

}  // namespace

// Offset or mask value i of a block's rows staged in LDS in the I/O dtype.
template <int DT>
__device__ __forceinline__ float staged(const unsigned char *lds, uint32_t i) {
  if constexpr (DT == DCN_F32) {
    return reinterpret_cast<const float *>(lds)[i];
  } else {
    return Io<DT>::lo((uint32_t) reinterpret_cast<const uint16_t *>(lds)[i]);
  }
}

// Untiled backward for any point set, stride and dilation: 16 lanes per
// pixel-group, one channel per lane (one DPP row), so each corner's gather is
// one request per pixel-group and its grad_input scatter one 64-byte atomic
// request of the row (a lane per channel: the hardware adds one fp32 per
// lane).  16-bit I/O (DT) reads its tensors as they are, computes in fp32,
// accumulates grad_input in an fp32 buffer of the input's shape and rounds
// grad_offset and grad_mask once to the I/O dtype.
template <int DT, int KH_, int KW_, bool SOFTMAX>
__global__ void __launch_bounds__(kBlock) dcn_bwd_kernel(BwdParams bp) {
  using io = Io<DT>;
  const FwdParams &p = bp.f;
  constexpr int CG = kGroupChannels;
  constexpr int BLOCK_PG = kBlock / CG;
  constexpr uint32_t EB = io::kBytes;
  constexpr uint32_t GX = 4 / EB;  // input byte offset -> fp32 grad_input byte offset
  constexpr bool FIXED = KH_ > 0;
  const int KH = FIXED ? KH_ : p.KH;
  const int KW = FIXED ? KW_ : p.KW;
  const int K = FIXED ? KH_ * KW_ : KH * KW - p.RC;  // fixed extents never drop the centre

  // LDS: the block's offset rows and mask rows (I/O dtype), then gm (fp32).
  extern __shared__ __align__(16) unsigned char lds[];
  const unsigned char *lds_off = lds;
  const unsigned char *lds_mask = lds + (uint32_t)BLOCK_PG * K * 2 * EB;
  float *lds_gm = reinterpret_cast<float *>(lds + (uint32_t)BLOCK_PG * K * 3 * EB);

  const uint32_t blk = xcd_block(blockIdx.x, gridDim.x);
  const uint32_t pg0 = blk * BLOCK_PG;
  const uint32_t npg = min((uint32_t)BLOCK_PG, p.pg_total - pg0);
  stage_to_lds(lds, static_cast<const unsigned char *>(p.offset) + (uint64_t)pg0 * K * 2 * EB, npg * K * 2 * EB);
  stage_to_lds(lds + (uint32_t)BLOCK_PG * K * 2 * EB,
               static_cast<const unsigned char *>(p.mask) + (uint64_t)pg0 * K * EB, npg * K * EB);
  __syncthreads();

  const uint32_t lp = threadIdx.x / CG;
  const uint32_t ch = threadIdx.x % CG;
  // The 16 lanes of a pixel-group (one DPP row) leave together, so the DPP
  // partners of a live lane are live.
  if (lp >= npg) return;
  const uint32_t pg = pg0 + lp;

  const uint32_t pix = fast_div(pg, p.div_g);
  const uint32_t g = pg - pix * (uint32_t)p.G;
  const uint32_t t = fast_div(pix, p.div_wo);
  const uint32_t wo = pix - t * (uint32_t)p.Wo;
  const uint32_t n = fast_div(t, p.div_ho);
  const uint32_t ho = t - n * (uint32_t)p.Ho;

  const uint32_t mrow = lp * K;
  float mx = 0.f, inv = 1.f;
  if constexpr (SOFTMAX) {
    mx = -INFINITY;
    for (int k = 0; k < K; ++k) mx = fmaxf(mx, staged<DT>(lds_mask, mrow + k));
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += __expf(staged<DT>(lds_mask, mrow + k) - mx);
    inv = __builtin_amdgcn_rcpf(sum);
  }
  auto weight = [&](int k) -> float {
    if constexpr (SOFTMAX) return __expf(staged<DT>(lds_mask, mrow + k) - mx) * inv;
    else return staged<DT>(lds_mask, mrow + k);
  };

  const float gy = io::one(bp.grad_out, (int64_t)pg * CG + ch);

  const uint32_t pix_bytes = (uint32_t)p.C * EB;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const uint32_t base = n * (uint32_t)p.H * row_bytes + (g * CG + ch) * EB;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const __amdgpu_buffer_rsrc_t rgx = make_rsrc(bp.grad_in, p.in_bytes * GX);
  const int by = (int)ho * p.SH - p.PH;
  const int bx = (int)wo * p.SW - p.PW;
  const float s = p.scale;
  unsigned char *goff = static_cast<unsigned char *>(bp.grad_offset) + (uint64_t)pg * K * 2 * EB;

  // One corner value of this lane's channel (0 at kOutOfRange).
  auto corner = [&](uint32_t a) -> float {
    if constexpr (DT == DCN_F32) {
      return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rin, (int)a, 0, 0));
    } else {
      return io::lo((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rin, (int)a, 0, 0));
    }
  };
  // grad_input offset of an input offset (fp32 elements; out of range stays so)
  auto gxo = [&](uint32_t a) -> int { return (int)(a == kOutOfRange ? kOutOfRange : a * GX); };

  // Point k at grid position (ii, jj).
  auto point = [&](const int ii, const int jj, const int k) {
    const float dx = s * staged<DT>(lds_off, (mrow + k) * 2);
    const float dy = s * staged<DT>(lds_off, (mrow + k) * 2 + 1);
    const bool nan_loc = (dx != dx) | (dy != dy);
    // Clamp first (|s*offset| >= 2^24 is far outside any map, and an infinite
    // offset must not turn the fraction into Inf - Inf), then split into an
    // integer part and an exact fraction in [0, 1).
    const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
    const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
    const float fx = floorf(cx), fy = floorf(cy);
    const float lx = cx - fx, ly = cy - fy;
    const int x0 = bx + jj * p.DW + (int)fx;
    const int y0 = by + ii * p.DH + (int)fy;
    const float mk = weight(k);
    const float hx = 1.f - lx, hy = 1.f - ly;

    // A NaN location reads and scatters nothing (its gradients are NaN).
    const bool vy0 = !nan_loc && (uint32_t)y0 < (uint32_t)p.H;
    const bool vy1 = !nan_loc && (uint32_t)(y0 + 1) < (uint32_t)p.H;
    const bool vx0 = (uint32_t)x0 < (uint32_t)p.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)p.W;
    const uint32_t a00r = base + (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_bytes;
    const uint32_t a00 = (vy0 && vx0) ? a00r : kOutOfRange;
    const uint32_t a01 = (vy0 && vx1) ? a00r + pix_bytes : kOutOfRange;
    const uint32_t a10 = (vy1 && vx0) ? a00r + row_bytes : kOutOfRange;
    const uint32_t a11 = (vy1 && vx1) ? a00r + row_bytes + pix_bytes : kOutOfRange;

    const float v00 = corner(a00), v01 = corner(a01), v10 = corner(a10), v11 = corner(a11);
    const float top = hx * v00 + lx * v01;  // row y0 along x
    const float bot = hx * v10 + lx * v11;  // row y0+1 along x
    const float gb = row16_sum(gy * (hy * top + ly * bot));
    const float gdy = row16_sum(gy * (bot - top));
    const float gdx = row16_sum(gy * (hy * (v01 - v00) + ly * (v11 - v10)));
    // Every lane of the row holds the totals: lane 0 keeps gm_k in the
    // pixel-group's LDS row and writes the offset gradient.
    if (ch == 0) {
      lds_gm[mrow + k] = nan_loc ? __builtin_nanf("") : gb;
      const float gox = nan_loc ? __builtin_nanf("") : s * mk * gdx;
      const float goy = nan_loc ? __builtin_nanf("") : s * mk * gdy;
      if constexpr (DT == DCN_F32) {
        reinterpret_cast<float2 *>(goff)[k] = make_float2(gox, goy);
      } else {
        reinterpret_cast<uint32_t *>(goff)[k] = io::pack(gox, goy);
      }
    }

    // Scatter m_k * w_corner * gy into grad_input (out-of-map corners carry
    // an offset beyond the buffer, and the hardware drops those atomics).
    const float g = mk * gy;
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(g * hy * hx, rgx, gxo(a00), 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(g * hy * lx, rgx, gxo(a01), 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(g * ly * hx, rgx, gxo(a10), 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(g * ly * lx, rgx, gxo(a11), 0, 0);
  };
  if constexpr (FIXED) {
#pragma unroll
    for (int ii = 0; ii < KH_; ++ii)
#pragma unroll
      for (int jj = 0; jj < KW_; ++jj) point(ii, jj, ii * KW_ + jj);
  } else {
    // Row-major over the grid; with RC the centre is skipped and the points
    // after it take the next indices.
    const int centre = p.RC ? (KH / 2) * KW + KW / 2 : -1;
    for (int q = 0, k = 0; q < KH * KW; ++q) {
      if (q == centre) continue;
      const int ii = q / KW;
      point(ii, q - ii * KW, k++);
    }
  }

  // grad_mask: raw gm_k for DCNv4, through the softmax Jacobian for DCNv3.
  // Lane ch of the row writes the points k = ch, ch + 16, ... (lane 0's LDS
  // writes above precede these reads in the wave's program order).
  float dot = 0.f;
  if constexpr (SOFTMAX) {
    for (int k = 0; k < K; ++k) dot = fmaf(weight(k), lds_gm[mrow + k], dot);
  }
  unsigned char *gmask = static_cast<unsigned char *>(bp.grad_mask) + (uint64_t)pg * K * EB;
  for (int k = (int)ch; k < K; k += CG) {
    const float gmk = lds_gm[mrow + k];
    const float v = SOFTMAX ? weight(k) * (gmk - dot) : gmk;
    if constexpr (DT == DCN_F32) {
      reinterpret_cast<float *>(gmask)[k] = v;
    } else {
      reinterpret_cast<uint16_t *>(gmask)[k] = (uint16_t)(io::pack(v, 0.f) & 0xffffu);
    }
  }
}

__global__ void __launch_bounds__(kBlock) dcn_zero_kernel(uint4 *dst, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = make_uint4(0, 0, 0, 0);
}

// dst[i] = round-to-nearest-even(src[i]) for 8 elements per lane and step.
template <int DT>
__global__ void __launch_bounds__(kBlock) dcn_narrow_kernel(const float4 *src, uint4 *dst, uint64_t n8) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += stride) {
    const float4 a = src[2 * i], b = src[2 * i + 1];
    dst[i] = make_uint4(Io<DT>::pack(a.x, a.y), Io<DT>::pack(a.z, a.w), Io<DT>::pack(b.x, b.y),
                        Io<DT>::pack(b.z, b.w));
  }
}

namespace {

template <int DT, int KH, int KW, bool SM>
hipError_t launch_one(const BwdParams &p, hipStream_t s) {
  constexpr int BLOCK_PG = kBlock / kGroupChannels;
  const int K = p.f.KH * p.f.KW - p.f.RC;
  const size_t lds = (size_t)BLOCK_PG * K * (3 * Io<DT>::kBytes + 4);
  const uint32_t blocks = (p.f.pg_total + BLOCK_PG - 1) / BLOCK_PG;
  hipLaunchKernelGGL((dcn_bwd_kernel<DT, KH, KW, SM>), dim3(blocks), dim3(kBlock), lds, s, p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_untiled(int softmax, const BwdParams &p, hipStream_t s) {
  if (p.f.KH == 3 && p.f.KW == 3 && !p.f.RC)
    return softmax ? launch_one<DT, 3, 3, true>(p, s) : launch_one<DT, 3, 3, false>(p, s);
  return softmax ? launch_one<DT, 0, 0, true>(p, s) : launch_one<DT, 0, 0, false>(p, s);
}

}  // namespace

// Backward path override for tests and measurements: DCN_MI355X_BWD_PATH =
// "generic" (untiled kernel), "tiled" (the half-window tiled kernel, fp32
// only), "quad" (the lane-quad tiled kernel, the default where it applies
// and the whole-map kernel does not) or "map" (the whole-map kernel, the
// default where it applies).  Read at every call.
bool backward_takes_map(const FwdParams &p) {
  const char *e = getenv("DCN_MI355X_BWD_PATH");
  if (e && (!strcmp(e, "generic") || !strcmp(e, "tiled") || !strcmp(e, "quad"))) return false;
  return backward_map_applies(p);
}

hipError_t launch_backward(int dtype, int softmax, const BwdParams &p, bool whole_map, hipStream_t s) {
  if (whole_map) return launch_backward_map(dtype, softmax, p, s);
  const char *e = getenv("DCN_MI355X_BWD_PATH");
  const bool generic = e && !strcmp(e, "generic");
  const bool halves = e && !strcmp(e, "tiled");
  if (!generic && !halves) {
    const hipError_t q = launch_backward_quad(dtype, softmax, p, s);
    if (q != hipErrorNotSupported) return q;
  }
  if (!generic && dtype == DCN_F32) {
    const hipError_t t = launch_backward_tiled(softmax, p, s);
    if (t != hipErrorNotSupported) return t;
  }
  switch (dtype) {
    case DCN_F32: return launch_untiled<DCN_F32>(softmax, p, s);
    case DCN_F16: return launch_untiled<DCN_F16>(softmax, p, s);
    case DCN_BF16: return launch_untiled<DCN_BF16>(softmax, p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero(void *dst, uint64_t bytes, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  uint64_t blocks = (n16 + kBlock - 1) / kBlock;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(dcn_zero_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, s,
                     static_cast<uint4 *>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_narrow(int dtype, const void *src, void *dst, uint64_t count, hipStream_t s) {
  const uint64_t n8 = count / 8;
  if (n8 == 0) return hipSuccess;
  uint64_t blocks = (n8 + kBlock - 1) / kBlock;
  if (blocks > 8192) blocks = 8192;
  const float4 *in = static_cast<const float4 *>(src);
  uint4 *out = static_cast<uint4 *>(dst);
  switch (dtype) {
    case DCN_F16: hipLaunchKernelGGL(dcn_narrow_kernel<DCN_F16>, dim3((uint32_t)blocks), dim3(kBlock), 0, s, in, out, n8); break;
    case DCN_BF16: hipLaunchKernelGGL(dcn_narrow_kernel<DCN_BF16>, dim3((uint32_t)blocks), dim3(kBlock), 0, s, in, out, n8); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dcn
