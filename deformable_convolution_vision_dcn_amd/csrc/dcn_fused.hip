// dcn_fused.hip -- the DCN core fused with the linear steps around it
// (wmrh.cn/news/61976, section 二):
//   GEN  -- steps 2 and 3: the offsets and the mask values of every point and
//           group come from two linear branches of a guide feature at the
//           output pixel, offset = guide W_off^T + b_off (rows ordered
//           (g, k, x|y)), mask = guide W_mask^T + b_mask (rows (g, k)); they
//           are formed in the kernel, kept in fp32 and never written out;
//   PROJ -- step 4: the weighted sum of every channel of a pixel goes through
//           the output_proj linear layer, out = y W_out^T + b_out (C x C),
//           before it is stored.
//
// Layout of the work: a block of 256 threads (four waves) owns PIX = 16 MT
// (16 or 32) consecutive output pixels and walks the groups in chunks of GC.  A chunk's
// LDS row holds its 2 K GC offset values, padded to a multiple of 16, then
// its K GC mask values, so that no 16-column tile mixes the two.
//   1. Generation (GEN): the chunk's offset and mask columns for the PIX
//      pixels, a GEMM of M = PIX, N = GC*K*3, K = Cgd on the matrix cores
//      (v_mfma_f32_16x16x4f32 for fp32, ..._16x16x32_bf16 / _f16 for 16-bit
//      I/O, fp32 accumulation).  Wave w takes the 16-column tiles w, w+4, ...
//      and all MT row tiles, so each weight fragment is loaded once per block
//      and used MT times; the k loop fetches the next step's fragments before
//      it issues this step's matrix instructions; the results (plus bias) land
//      in LDS.  Without GEN
//      the chunk's offset and mask rows are copied into the same LDS layout.
//   2. Sampling: four lanes per pixel-group (four channels each) read the
//      pixel-group's offsets and logits from LDS, form the softmax (DCNv3),
//      locations and bilinear weights and gather the four corners of every
//      point from the input with raw buffer loads (a corner off the map
//      carries an offset beyond the buffer and reads 0).
//   3. Projection (PROJ): the PIX x C core output stays in LDS (fp32) and a
//      second GEMM (M = PIX, N = C, K = C) applies W_out.  For 16-bit I/O the
//      fp32 core output enters the 16-bit matrix cores as two parts, its
//      rounding hi to the I/O dtype and the rounding of y - hi, so that the
//      product sees about twice the dtype's significant bits.
// Fragments: in the 16x16 MFMA shapes lane l holds row (l mod 16) of A and
// column (l mod 16) of B at k = k0 + KL (l / 16) + e, e < KL (KL = 4 values
// for fp32, which feeds four k = 4 instructions, 8 for 16-bit), i.e. 16
// contiguous bytes of a row-major operand; result register v of lane l is
// row 4 (l / 16) + v, column l mod 16.  The order of the k terms inside a
// 16-value step is a permutation of the plain order, which leaves the sum
// unchanged up to rounding.
#include <algorithm>

#include "dcn_device.hpp"

namespace dcn {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Largest block, in 16-pixel row tiles: the generation GEMM is fastest with
// 32 pixels (64 need 253 VGPRs and one wave per SIMD), the projection with
// 16 (measured at the InternImage-L stage shapes).
#ifndef DCN_FUSED_MAX_MT_GEN
#define DCN_FUSED_MAX_MT_GEN 2
#endif
#ifndef DCN_FUSED_MAX_MT_PROJ
#define DCN_FUSED_MAX_MT_PROJ 1
#endif

constexpr int kFusedThreads = 256;
constexpr int kFusedTilesPerWave = 4;  // 16-column tiles per wave in one generation chunk

// One k step of the 16x16 MFMA shapes: the lane's 16-byte A and B fragments.
template <int DT>
struct Mma {
  static constexpr int kPerLane = DT == DCN_F32 ? 4 : 8;  // k values of one lane per step
  static constexpr int kStep = 4 * kPerLane;               // k per step (four lane rows of 16)
  __device__ static __forceinline__ f32x4 mac(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DT == DCN_F32) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[t]), __uint_as_float(b[t]), c, 0, 0, 0);
      return c;
    } else if constexpr (DT == DCN_BF16) {
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                     c, 0, 0, 0);
    } else {
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                    0, 0, 0);
    }
  }
};

__host__ __device__ constexpr int pad16(int v) { return (v + 15) & ~15; }

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

}  // namespace

template <int DT, bool SOFTMAX, bool GEN, bool PROJ, int MT>
__global__ void __launch_bounds__(kFusedThreads) dcn_fused_kernel(FusedParams fp) {
  using io = Io<DT>;
  using mma = Mma<DT>;
  constexpr int PIX = 16 * MT;
  constexpr int CG = kGroupChannels;
  constexpr uint32_t EB = io::kBytes;
  const FwdParams &p = fp.f;
  const int K = p.KH * p.KW - p.RC;
  const int G = p.G, C = p.C;
  const int GC = fp.gc;           // groups per chunk
  const int RS = pad16(GC * K * 2) + GC * K;  // LDS row stride of a chunk's columns (floats)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;

  extern __shared__ __align__(16) float lds[];
  float *om = lds;                 // [PIX][RS]: offsets of the chunk, then its mask values
  float *ys = lds + PIX * RS;      // [PIX][C]: the core output (PROJ)

  const uint32_t pix0 = xcd_block(blockIdx.x, gridDim.x) * PIX;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const float s = p.scale;

  for (int g0 = 0; g0 < G; g0 += GC) {
    const int gc = min(GC, G - g0);
    const int n_off = gc * K * 2, n_msk = gc * K;  // offset and mask values of the chunk
    const int m0 = pad16(n_off);                   // LDS column of the first mask value

    if constexpr (GEN) {
      // om[r][col] = guide[pix0 + r] . W[row(col)] + bias[row(col)]
      const __amdgpu_buffer_rsrc_t rg = make_rsrc(fp.guide, fp.guide_bytes);
      const __amdgpu_buffer_rsrc_t rwo = make_rsrc(fp.w_off, fp.w_off_bytes);
      const __amdgpu_buffer_rsrc_t rwm = make_rsrc(fp.w_mask, fp.w_mask_bytes);
      const int cgd = fp.cgd;
      const int ntiles = (m0 + n_msk + 15) / 16;
      f32x4 acc[kFusedTilesPerWave][MT];
#pragma unroll
      for (int j = 0; j < kFusedTilesPerWave; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[j][m] = f32x4{0.f, 0.f, 0.f, 0.f};
      // this lane's B column of each of the wave's tiles, as a weight row;
      // a tile is all offset columns or all mask columns (wave-uniform)
      uint32_t wrow[kFusedTilesPerWave];
      bool in_off[kFusedTilesPerWave], live[kFusedTilesPerWave];
#pragma unroll
      for (int j = 0; j < kFusedTilesPerWave; ++j) {
        const int col = (wave + 4 * j) * 16 + lr;
        in_off[j] = (wave + 4 * j) * 16 < m0;
        live[j] = in_off[j] ? col < n_off : col - m0 < n_msk;
        wrow[j] = in_off[j] ? (uint32_t)(g0 * K * 2 + col) : (uint32_t)(g0 * K + (col - m0));
      }
      // The k loop is software-pipelined: the fragments of step k0 + kStep
      // are requested before the matrix instructions of step k0 issue.
      u32x4 a[MT], b[kFusedTilesPerWave];
      auto fetch = [&](int k0, u32x4 (&fa)[MT], u32x4 (&fb)[kFusedTilesPerWave]) {
        const int kk = k0 + mma::kPerLane * lq;
        const bool kok = kk < cgd;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint32_t q = pix0 + 16 * m + lr;
          fa[m] = load16(rg, kok && q < fp.npix ? (q * (uint32_t)cgd + kk) * EB : kOutOfRange);
        }
#pragma unroll
        for (int j = 0; j < kFusedTilesPerWave; ++j) {
          const uint32_t voff =
              kok && live[j] && wave + 4 * j < ntiles ? (wrow[j] * (uint32_t)cgd + kk) * EB : kOutOfRange;
          fb[j] = in_off[j] ? load16(rwo, voff) : load16(rwm, voff);
        }
      };
      fetch(0, a, b);
      for (int k0 = 0; k0 < cgd; k0 += mma::kStep) {
        u32x4 an[MT], bn[kFusedTilesPerWave];
        fetch(k0 + mma::kStep, an, bn);  // past the last step: every offset out of range, nothing read
#pragma unroll
        for (int j = 0; j < kFusedTilesPerWave; ++j) {
          if (wave + 4 * j >= ntiles) break;  // wave-uniform
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[j][m] = mma::mac(a[m], b[j], acc[j][m]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) a[m] = an[m];
#pragma unroll
        for (int j = 0; j < kFusedTilesPerWave; ++j) b[j] = bn[j];
      }
#pragma unroll
      for (int j = 0; j < kFusedTilesPerWave; ++j) {
        const int col = (wave + 4 * j) * 16 + lr;
        if (wave + 4 * j >= ntiles || !live[j]) continue;
        float bias = 0.f;
        if (in_off[j] && fp.b_off) bias = io::one(fp.b_off, wrow[j]);
        if (!in_off[j] && fp.b_mask) bias = io::one(fp.b_mask, wrow[j]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) om[(16 * m + 4 * lq + v) * RS + col] = acc[j][m][v] + bias;
      }
    } else {
      // the chunk's offset and mask rows, widened to fp32, in the same layout
      const int per_px = n_off + n_msk;
      for (int e = threadIdx.x; e < PIX * per_px; e += kFusedThreads) {
        const int r = e / per_px, col = e - r * per_px;
        const uint32_t q = pix0 + r;
        float v = 0.f;
        if (q < fp.npix) {
          if (col < n_off) {
            v = io::one(p.offset, ((int64_t)q * G + g0) * K * 2 + col);
          } else {
            v = io::one(p.mask, ((int64_t)q * G + g0) * K + (col - n_off));
          }
        }
        om[r * RS + (col < n_off ? col : m0 + (col - n_off))] = v;
      }
    }
    __syncthreads();  // the chunk's offsets and mask values are in LDS

    // Sampling: four lanes per pixel-group, pixel-groups pixel-major.
    {
      const int sub = threadIdx.x & 3;
      for (int t = threadIdx.x >> 2; t < PIX * gc; t += kFusedThreads / 4) {
        const int px = t / gc, gl = t - px * gc;
        const uint32_t q = pix0 + px;
        if (q >= fp.npix) break;  // pixel-major: every later t is past the end too
        const int g = g0 + gl;
        const float *ro = om + px * RS + gl * K * 2;
        const float *rm = om + px * RS + m0 + gl * K;
        float mx = 0.f, inv = 1.f;
        if constexpr (SOFTMAX) {
          mx = -INFINITY;
          for (int k = 0; k < K; ++k) mx = fmaxf(mx, rm[k]);
          float sum = 0.f;
          for (int k = 0; k < K; ++k) sum += __expf(rm[k] - mx);
          inv = __builtin_amdgcn_rcpf(sum);
        }
        const uint32_t tq = fast_div(q, p.div_wo);
        const uint32_t wo = q - tq * (uint32_t)p.Wo;
        const uint32_t n = fast_div(tq, p.div_ho);
        const uint32_t ho = tq - n * (uint32_t)p.Ho;
        const uint32_t pix_bytes = (uint32_t)C * EB, row_bytes = (uint32_t)p.W * pix_bytes;
        const uint32_t base = n * (uint32_t)p.H * row_bytes + (uint32_t)(g * CG + 4 * sub) * EB;
        const int by = (int)ho * p.SH - p.PH, bx = (int)wo * p.SW - p.PW;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        bool nan_loc = false;
        const int centre = p.RC ? (p.KH / 2) * p.KW + p.KW / 2 : -1;
        for (int qg = 0, k = 0; qg < p.KH * p.KW; ++qg) {
          if (qg == centre) continue;
          const int ii = qg / p.KW, jj = qg - ii * p.KW;
          const float dx = s * ro[2 * k], dy = s * ro[2 * k + 1];
          nan_loc |= (dx != dx) | (dy != dy);
          const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
          const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
          const float fx = floorf(cx), fy = floorf(cy);
          const float lx = cx - fx, ly = cy - fy;
          const int x0 = bx + jj * p.DW + (int)fx, y0 = by + ii * p.DH + (int)fy;
          const float mk = SOFTMAX ? __expf(rm[k] - mx) * inv : rm[k];
          const float wy1 = ly * mk, wy0 = mk - wy1;
          const float w01 = wy0 * lx, w00 = wy0 - w01, w11 = wy1 * lx, w10 = wy1 - w11;
          const bool vy0 = (uint32_t)y0 < (uint32_t)p.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)p.H;
          const bool vx0 = (uint32_t)x0 < (uint32_t)p.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)p.W;
          const uint32_t a00 = base + (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_bytes;
          constexpr int NW = 4 * EB / 4;
          uint32_t q00[NW], q01[NW], q10[NW], q11[NW];
          buffer_load_words<NW>(rin, vy0 && vx0 ? a00 : kOutOfRange, q00);
          buffer_load_words<NW>(rin, vy0 && vx1 ? a00 + pix_bytes : kOutOfRange, q01);
          buffer_load_words<NW>(rin, vy1 && vx0 ? a00 + row_bytes : kOutOfRange, q10);
          buffer_load_words<NW>(rin, vy1 && vx1 ? a00 + row_bytes + pix_bytes : kOutOfRange, q11);
          float v00[4], v01[4], v10[4], v11[4];
          unpack<DT, NW>(q00, v00);
          unpack<DT, NW>(q01, v01);
          unpack<DT, NW>(q10, v10);
          unpack<DT, NW>(q11, v11);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[c] = fmaf(w00, v00[c], acc[c]);
            acc[c] = fmaf(w01, v01[c], acc[c]);
            acc[c] = fmaf(w10, v10[c], acc[c]);
            acc[c] = fmaf(w11, v11[c], acc[c]);
          }
          ++k;
        }
        if (nan_loc) {
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = __builtin_nanf("");
        }
        if constexpr (PROJ) {
          *reinterpret_cast<float4 *>(ys + px * C + g * CG + 4 * sub) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
          uint32_t w[4 * EB / 4];
          pack_words<DT, 4>(acc, w);
          store_words<4 * EB / 4>(static_cast<unsigned char *>(p.output) + ((uint64_t)q * C + g * CG + 4 * sub) * EB,
                                  w);
        }
      }
    }
    __syncthreads();  // every read of the chunk's LDS columns is done
  }

  if constexpr (PROJ) {
    // out[pix0 + r][col] = ys[r] . W_out[col] + b_out[col]
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(fp.w_out, fp.w_out_bytes);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(p.output, p.out_bytes);
    const int ntiles = C / 16;
    for (int nt = wave; nt < ntiles; nt += 4) {
      const int col = nt * 16 + lr;
      f32x4 acc[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      // B fragments one step ahead (software-pipelined), A from LDS
      auto fetch_b = [&](int k0) {
        const int kk = k0 + mma::kPerLane * lq;
        return load16(rw, kk < C ? ((uint32_t)col * (uint32_t)C + kk) * EB : kOutOfRange);
      };
      u32x4 bnext = fetch_b(0);
      for (int k0 = 0; k0 < C; k0 += mma::kStep) {
        const int kk = k0 + mma::kPerLane * lq;
        const bool kok = kk < C;  // C is a multiple of 16, the 16-bit step 32
        const u32x4 b = bnext;
        bnext = fetch_b(k0 + mma::kStep);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float *src = ys + (16 * m + lr) * C + (kok ? kk : 0);
          if constexpr (DT == DCN_F32) {
            const float4 v = kok ? *reinterpret_cast<const float4 *>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
            const u32x4 a{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
            acc[m] = mma::mac(a, b, acc[m]);
          } else {  // y = hi + lo, each part in the I/O dtype
            float y[8];
            const float4 v0 = kok ? *reinterpret_cast<const float4 *>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 v1 = kok ? *reinterpret_cast<const float4 *>(src + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
            y[0] = v0.x, y[1] = v0.y, y[2] = v0.z, y[3] = v0.w, y[4] = v1.x, y[5] = v1.y, y[6] = v1.z, y[7] = v1.w;
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              hi[e] = io::pack(y[2 * e], y[2 * e + 1]);
              lo[e] = io::pack(y[2 * e] - io::lo(hi[e]), y[2 * e + 1] - io::hi(hi[e]));
            }
            acc[m] = mma::mac(u32x4{hi[0], hi[1], hi[2], hi[3]}, b, acc[m]);
            acc[m] = mma::mac(u32x4{lo[0], lo[1], lo[2], lo[3]}, b, acc[m]);
          }
        }
      }
      const float bias = fp.b_out ? io::one(fp.b_out, col) : 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t q = pix0 + 16 * m + 4 * lq + v;
          const float val = acc[m][v] + bias;
          const uint32_t at = q < fp.npix ? ((uint32_t)q * (uint32_t)C + col) * EB : kOutOfRange;
          if constexpr (DT == DCN_F32) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), rout, (int)at, 0, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(io::pack(val, 0.f) & 0xffffu), rout, (int)at, 0, 0);
          }
        }
    }
  }
}

namespace {

// Groups per chunk: at most four 16-column tiles per wave (the padded row of
// 2 K GC offset and K GC mask columns at most 256), the chunks of one call
// as even as possible.
int fused_groups_per_chunk(int G, int K) {
  int cap = 1;
  while (cap < G && pad16(2 * K * (cap + 1)) + K * (cap + 1) <= 16 * 4 * kFusedTilesPerWave) ++cap;
  const int chunks = (G + cap - 1) / cap;
  return (G + chunks - 1) / chunks;
}

size_t fused_lds_bytes(int mt, int gc, int K, int C, bool proj) {
  return (size_t)16 * mt * ((size_t)pad16(gc * K * 2) + (size_t)gc * K + (proj ? (size_t)C : 0)) * sizeof(float);
}

constexpr size_t kFusedLdsLimit = 160 * 1024;

template <int DT, bool SM, bool GEN, bool PROJ, int MT>
hipError_t launch_fused_mt(const FusedParams &fp, size_t lds, hipStream_t s) {
  auto kern = dcn_fused_kernel<DT, SM, GEN, PROJ, MT>;
  const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFusedLdsLimit);
  if (attr != hipSuccess) return attr;
  const uint32_t blocks = (fp.npix + 16 * MT - 1) / (16 * MT);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kFusedThreads), lds, s, fp);
  return hipGetLastError();
}

template <int DT, bool SM, bool GEN, bool PROJ>
hipError_t launch_fused_dt(FusedParams fp, hipStream_t s) {
  const int K = fp.f.KH * fp.f.KW - fp.f.RC;
  fp.gc = fused_groups_per_chunk(fp.f.G, K);
  // the most pixels per block (weights reused the most) whose LDS fits
  for (int mt : {4, 2, 1}) {
    const size_t lds = fused_lds_bytes(mt, fp.gc, K, fp.f.C, PROJ);
    if (mt > (PROJ ? DCN_FUSED_MAX_MT_PROJ : DCN_FUSED_MAX_MT_GEN) || lds > kFusedLdsLimit) continue;
    if (mt == 4) return launch_fused_mt<DT, SM, GEN, PROJ, 4>(fp, lds, s);
    if (mt == 2) return launch_fused_mt<DT, SM, GEN, PROJ, 2>(fp, lds, s);
    return launch_fused_mt<DT, SM, GEN, PROJ, 1>(fp, lds, s);
  }
  return hipErrorNotSupported;
}

template <bool GEN, bool PROJ>
hipError_t launch_fused_any(int dtype, int softmax, const FusedParams &fp, hipStream_t s) {
  switch (dtype) {
    case DCN_F32:
      return softmax ? launch_fused_dt<DCN_F32, true, GEN, PROJ>(fp, s) : launch_fused_dt<DCN_F32, false, GEN, PROJ>(fp, s);
    case DCN_F16:
      return softmax ? launch_fused_dt<DCN_F16, true, GEN, PROJ>(fp, s) : launch_fused_dt<DCN_F16, false, GEN, PROJ>(fp, s);
    case DCN_BF16:
      return softmax ? launch_fused_dt<DCN_BF16, true, GEN, PROJ>(fp, s)
                     : launch_fused_dt<DCN_BF16, false, GEN, PROJ>(fp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// True when the fused kernel's LDS fits for this problem (16 pixels per
// block at least).
bool fused_fits(int G, int K, int C, bool proj) {
  return fused_lds_bytes(1, fused_groups_per_chunk(G, K), K, C, proj) <= kFusedLdsLimit;
}

hipError_t launch_forward_generated(int dtype, int softmax, const FusedParams &fp, hipStream_t s) {
  return launch_fused_any<true, false>(dtype, softmax, fp, s);
}

hipError_t launch_forward_projected(int dtype, int softmax, const FusedParams &fp, hipStream_t s) {
  return launch_fused_any<false, true>(dtype, softmax, fp, s);
}

}  // namespace dcn
