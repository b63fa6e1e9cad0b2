// dcn_bwd_tile.hip -- LDS-tiled gfx950 backward kernel of the DCN core (fp32)
// for 3x3 kernel points at stride 1 and dilation 1 (the InternImage
// configuration; wmrh.cn/news/61976, section 二 steps 2-4 and section 三).
//
// The derivatives are those of the untiled backward kernel: every in-map
// corner of a sample receives m_k * w_corner * gy_c; the offset gradient is
// s * m_k * sum_c gy_c * dB_k[c]/d(px, py) (one-sided from the right at integer
// coordinates); the mask gradient is gm_k = sum_c gy_c * B_k[c], through the
// softmax Jacobian for DCNv3.
//
// Why tiles: the grad_input scatter is 576 fp32 additions per pixel-group
// (9 points x 4 corners x 16 channels) at offset-driven addresses.  Sent to
// global memory one by one they are scattered atomics that the L2 serialises.
// Here a block owns one (image, 16x16 output tile, group) work item, one lane
// per pixel-group, and
//   * stages the input window its samples can reach (the tile's 3x3 footprint
//     plus a halo of R pixels for the offsets) in LDS, to read the corners;
//   * accumulates the scatter into a second LDS window with LDS float
//     atomics, and adds that window to grad_input once at the end with
//     coalesced global atomics (16 channels of neighbouring pixels in
//     consecutive lanes), skipping the zeros;
//   * keeps the per-point channel sums (gm, d/dx, d/dy) of its pixel-group in
//     registers, so the offset and mask gradients need no cross-lane step.
// The 16 channels of a group go through LDS as two halves of 8 (32 bytes per
// window pixel), which keeps the two windows at 79 KB (halo 8) and two blocks
// per CU.
// Samples whose corners leave the window (|s * offset| beyond the halo) take
// the global path behind a wave ballot: buffer loads for the corners and
// buffer atomics for the scatter, the buffer range check turning corners
// outside the map into zeros and dropped additions.
#include "dcn_device.hpp"

namespace dcn {

constexpr int kBwdTile = 16;
#ifndef DCN_BWD_HALO
#define DCN_BWD_HALO 8
#endif
constexpr int kBwdHalo = DCN_BWD_HALO;
constexpr int kBwdSpan = kBwdTile + 2 * kBwdHalo + 3;     // window edge, pixels
constexpr int kBwdPixB = 32;                              // 8 fp32 channels
constexpr int kBwdRow = kBwdSpan * kBwdPixB;              // LDS bytes per window row
constexpr int kBwdSink = kBwdSpan * kBwdSpan * kBwdPixB;  // zero rows / sink rows
constexpr int kBwdWinBytes = kBwdSink + kBwdRow + 2 * kBwdPixB;
constexpr int kBwdThreads = kBwdTile * kBwdTile;

namespace {

__device__ __forceinline__ void lds_read16(const unsigned char *src, float (&v)[4]) {
  const float4 q = *reinterpret_cast<const float4 *>(src);
  v[0] = q.x;
  v[1] = q.y;
  v[2] = q.z;
  v[3] = q.w;
}

// Two neighbouring channels' fixed-point terms added by one 64-bit LDS
// integer add (ds_add_u64).  Float adds in LDS run at a small fraction of the
// integer rate on this chip, so the scatter accumulates in fixed point; a
// 64-bit add moves two channels for about the cost of one 32-bit add.  The
// pair is the 64-bit integer hi * 2^32 + lo (lo sign-extended into the high
// word), so a sum of such terms is (sum hi) * 2^32 + sum lo exactly, and as
// long as |sum lo| < 2^31 both sums are recovered from it (see unpack_pair).
__device__ __forceinline__ void lds_iadd2(unsigned char *dst, int lo, int hi) {
  const uint64_t v = ((uint64_t)(uint32_t)(hi + (lo >> 31)) << 32) | (uint32_t)lo;
  __hip_atomic_fetch_add(reinterpret_cast<uint64_t *>(dst), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// (sum lo, sum hi) of a pair accumulated by lds_iadd2.
__device__ __forceinline__ int2 unpack_pair(uint64_t v) {
  const int lo = (int)(uint32_t)v;
  const int hi = (int)((int64_t)(v - (uint64_t)(int64_t)lo) >> 32);
  return make_int2(lo, hi);
}

}  // namespace

template <bool SOFTMAX>
__global__ void __launch_bounds__(kBwdThreads, 2) dcn_bwd_tile_kernel(BwdParams bp, TileGeom tg) {
  const FwdParams &p = bp.f;
  constexpr int TS = kBwdTile, R = kBwdHalo, SPAN_W = kBwdSpan;
  constexpr int SPAN = SPAN_W * SPAN_W;
  constexpr int PIXB = kBwdPixB, ROW = kBwdRow, SINK = kBwdSink;
  constexpr int LIM = SPAN_W - 2;
  constexpr int CG = kGroupChannels, CH = CG / 2;  // channels per half
  constexpr int K = 9;
  constexpr int STAGERS = kBwdThreads / 2;  // two lanes (16 bytes each) per window pixel
  constexpr int SLOTS = (SPAN + STAGERS - 1) / STAGERS;
  constexpr int WAVES = kBwdThreads / 64;

  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *win = lds;                  // input half-window, then zero rows
  unsigned char *gwin = lds + kBwdWinBytes;  // fixed-point grad half-window, then sink rows
  float *wave_sums = reinterpret_cast<float *>(lds + 2 * kBwdWinBytes);

  const uint32_t lane = threadIdx.x;
  const int oy = (int)lane / TS, ox = (int)lane % TS;
  const uint32_t pix_bytes = (uint32_t)p.C * 4u;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const __amdgpu_buffer_rsrc_t rgx = make_rsrc(bp.grad_in, p.in_bytes);
  const float s = p.scale;

  // Work item -> (n, tile, g), g fastest.
  const uint32_t item = xcd_block(blockIdx.x, gridDim.x);
  const uint32_t tq = fast_div(item, tg.div_g);
  const uint32_t g = item - tq * (uint32_t)p.G;
  const uint32_t n = fast_div(tq, tg.div_tiles);
  const uint32_t tile_id = tq - n * (uint32_t)tg.tiles_per_img;
  const uint32_t tyi = fast_div(tile_id, tg.div_tiles_x);
  const uint32_t txi = tile_id - tyi * (uint32_t)tg.tiles_x;
  const int r0 = (int)tyi * TS, c0 = (int)txi * TS;
  const int Y0 = r0 - p.PH - R, X0 = c0 - p.PW - R;  // window origin
  const int ho = r0 + oy, wo = c0 + ox;
  const bool live = ho < p.Ho && wo < p.Wo;
  const uint32_t pg = live ? (((n * (uint32_t)p.Ho + ho) * (uint32_t)p.Wo + wo) * (uint32_t)p.G) + g : 0u;
  const uint32_t img = n * (uint32_t)p.H * row_bytes;

  // Zero rows after the input window (read by samples outside it).
  for (int z = (int)lane * 16; z < ROW + 2 * PIXB; z += kBwdThreads * 16)
    *reinterpret_cast<uint4 *>(win + SINK + z) = make_uint4(0, 0, 0, 0);

  // Own pixel-group: offsets and logits (a dead lane reads group 0).
  float off[2 * K], m[K];
  {
    // 18 floats at a 72-byte pitch: 8-byte aligned, so read as float2.
    const float2 *o2 = reinterpret_cast<const float2 *>(static_cast<const float *>(p.offset) + (uint64_t)pg * 2 * K);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float2 v = o2[k];
      off[2 * k] = v.x;
      off[2 * k + 1] = v.y;
    }
    const float *mk = static_cast<const float *>(p.mask) + (uint64_t)pg * K;
#pragma unroll
    for (int k = 0; k < K; ++k) m[k] = mk[k];
  }
  if constexpr (SOFTMAX) {
    float mx = m[0];
#pragma unroll
    for (int k = 1; k < K; ++k) mx = fmaxf(mx, m[k]);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      m[k] = __expf(m[k] - mx);
      sum += m[k];
    }
    const float inv = __builtin_amdgcn_rcpf(sum);
#pragma unroll
    for (int k = 0; k < K; ++k) m[k] *= inv;
  }
  float msum = 0.f;  // sum_k |m_k|: bounds what this pixel-group scatters per channel
#pragma unroll
  for (int k = 0; k < K; ++k) msum += fabsf(m[k]);

  float gb[K], gdx[K], gdy[K];
#pragma unroll
  for (int k = 0; k < K; ++k) gb[k] = gdx[k] = gdy[k] = 0.f;

  const uint32_t sq = lane / 2, sc = lane % 2;
  constexpr int NP = CH / 2;  // channel pairs per half
  int cro[NP];  // byte offset of channel pair (q + lane) mod 4 within a pixel slice
#pragma unroll
  for (int q = 0; q < NP; ++q) cro[q] = (int)(((uint32_t)q + lane) % NP) * 8;
#pragma unroll 1
  for (int h = 0; h < 2; ++h) {
    const uint32_t chan = (g * CG + h * CH + sc * 4) * 4u;  // this stager's 16 bytes
    // The sample locations are recomputed per half (an opaque copy of the
    // scale keeps the compiler from hoisting all nine points' state out of
    // this loop, which would not fit the register budget).
    float sh = s;
    asm volatile("" : "+v"(sh));
    // grad_out of the own pixel-group, this half's 8 channels.
    float gyh[CH];
    {
      const float4 *g4 = reinterpret_cast<const float4 *>(static_cast<const float *>(bp.grad_out) +
                                                          (uint64_t)pg * CG + h * CH);
#pragma unroll
      for (int q = 0; q < CH / 4; ++q) {
        const float4 v = g4[q];
        gyh[4 * q] = v.x;
        gyh[4 * q + 1] = v.y;
        gyh[4 * q + 2] = v.z;
        gyh[4 * q + 3] = v.w;
      }
    }
    // The same 8 values with their channel pairs rotated by this lane's
    // position: (gyr[2q], gyr[2q + 1]) = pair (q + lane) mod 4 (a 2-step
    // barrel rotation), for the bank-spread scatter below.
    float gyr[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) gyr[c] = gyh[c];
#pragma unroll
    for (int rs = 1; rs < NP; rs <<= 1) {
      const bool on = (lane & (uint32_t)rs) != 0;
      float t[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) t[c] = on ? gyr[(c + 2 * rs) % CH] : gyr[c];
#pragma unroll
      for (int c = 0; c < CH; ++c) gyr[c] = t[c];
    }

    // Fixed-point scale of this half-window.  Every window pixel-channel
    // receives at most the sum over the tile's pixel-groups of
    // sum_k |m_k| * max_c |gy_c| (the four corner weights of a sample are
    // non-negative and add up to 1), call it B.  With S = 2^(30 - e), B <= 2^e,
    // every partial sum of the scaled terms stays within 2^30, so the LDS
    // integer adds (two channels per 64-bit add) sum them exactly; each term
    // is rounded to the nearest multiple of 1/S.  A non-finite B (NaN or Inf
    // in grad_out or the mask), or a spread above 2^12 between B and the
    // smallest nonzero per-pixel-group bound (so that rounding to the tile's
    // grid stays small against every contributor), switches the half to fp32
    // global atomics.
    float gmax = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) gmax = fmaxf(gmax, fabsf(gyh[c]));
    // fmaxf drops NaN: a NaN in gy must still reach the bound
    float bound = live ? msum * gmax : 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) bound += live ? 0.f * gyh[c] : 0.f;
    float lmin = bound > 0.f ? bound : INFINITY;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      bound += __shfl_xor(bound, d, 64);
      lmin = fminf(lmin, __shfl_xor(lmin, d, 64));
    }

    __syncthreads();  // the previous half's flush has read gwin, every read of win is done
    if ((lane & 63) == 0) {
      wave_sums[lane / 64] = bound;
      wave_sums[WAVES + lane / 64] = lmin;
    }
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const int idx = (int)sq + u * STAGERS;
      const int sy = idx / SPAN_W, sx = idx - sy * SPAN_W;
      const int gy_ = Y0 + sy, gx_ = X0 + sx;
      const bool ok = idx < SPAN && (uint32_t)gy_ < (uint32_t)p.H && (uint32_t)gx_ < (uint32_t)p.W;
      uint32_t w[4];
      buffer_load_words<4>(rin, ok ? img + (uint32_t)gy_ * row_bytes + (uint32_t)gx_ * pix_bytes + chan : kOutOfRange, w);
      if (idx < SPAN) {
        *reinterpret_cast<uint4 *>(win + idx * PIXB + sc * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4 *>(gwin + idx * PIXB + sc * 16) = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();  // both half-windows and the wave bounds are ready

    float B = 0.f, bmin = INFINITY;
#pragma unroll
    for (int wv = 0; wv < WAVES; ++wv) {
      B += wave_sums[wv];
      bmin = fminf(bmin, wave_sums[WAVES + wv]);
    }
    // false for Inf and NaN, and for a spread above 2^12 (block-uniform)
    const bool fixed = B <= 3.0e38f && B <= kFixedSpread * bmin;
    int e = 0;
    frexpf(B, &e);
    e = e < -96 ? -96 : e;
    const float S = ldexpf(1.f, 30 - e), invS = ldexpf(1.f, e - 30);

#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = k / 3, j = k % 3;
      const float dx = sh * off[2 * k], dy = sh * off[2 * k + 1];
      const bool nan_loc = (dx != dx) | (dy != dy);
      const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
      const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
      const float fx = floorf(cx), fy = floorf(cy);
      const float lx = cx - fx, ly = cy - fy;
      const float hx = 1.f - lx, hy = 1.f - ly;
      const int ty = oy + i + R + (int)fy, tx = ox + j + R + (int)fx;  // window coordinates
      const bool inside = live && !nan_loc && (uint32_t)ty <= (uint32_t)LIM && (uint32_t)tx <= (uint32_t)LIM;
      const int A = inside ? ty * ROW + tx * PIXB : SINK;
      const float mk = m[k];
      const float w00 = mk * hy * hx, w01 = mk * hy * lx, w10 = mk * ly * hx, w11 = mk * ly * lx;
      const int y0 = Y0 + ty, x0 = X0 + tx;
      const bool vy0 = (uint32_t)y0 < (uint32_t)p.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)p.H;
      const bool vx0 = (uint32_t)x0 < (uint32_t)p.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)p.W;
      const uint32_t a = img + (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_bytes + (g * CG + h * CH) * 4u;

      // Per-corner dot products with grad_out: G_corner = sum_c gy_c v_corner[c].
      // The three sums follow from them (B_k is linear in the corners):
      //   gm = hy (hx G00 + lx G01) + ly (hx G10 + lx G11)
      //   d/dy = (hx G10 + lx G11) - (hx G00 + lx G01)
      //   d/dx = hy (G01 - G00) + ly (G11 - G10)
      float G00 = 0.f, G01 = 0.f, G10 = 0.f, G11 = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float v00[4], v01[4], v10[4], v11[4];
        lds_read16(win + A + t * 16, v00);
        lds_read16(win + A + PIXB + t * 16, v01);
        lds_read16(win + A + ROW + t * 16, v10);
        lds_read16(win + A + ROW + PIXB + t * 16, v11);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float gc = gyh[4 * t + c];
          G00 = fmaf(gc, v00[c], G00);
          G01 = fmaf(gc, v01[c], G01);
          G10 = fmaf(gc, v10[c], G10);
          G11 = fmaf(gc, v11[c], G11);
        }
      }
      // Corners outside the window but touching the map: global loads
      // (rare; skipped by the wave when no lane needs it).
      const bool fb = live && !inside && !nan_loc && (uint32_t)(y0 + 1) <= (uint32_t)p.H &&
                      (uint32_t)(x0 + 1) <= (uint32_t)p.W;
      const uint32_t a00 = (vy0 && vx0) ? a : kOutOfRange;
      const uint32_t a01 = (vy0 && vx1) ? a + pix_bytes : kOutOfRange;
      const uint32_t a10 = (vy1 && vx0) ? a + row_bytes : kOutOfRange;
      const uint32_t a11 = (vy1 && vx1) ? a + row_bytes + pix_bytes : kOutOfRange;
      if (__builtin_amdgcn_ballot_w64(fb) != 0) {
        if (fb) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            uint32_t q00[4], q01[4], q10[4], q11[4];
            buffer_load_words<4>(rin, a00 == kOutOfRange ? kOutOfRange : a00 + 16u * t, q00);
            buffer_load_words<4>(rin, a01 == kOutOfRange ? kOutOfRange : a01 + 16u * t, q01);
            buffer_load_words<4>(rin, a10 == kOutOfRange ? kOutOfRange : a10 + 16u * t, q10);
            buffer_load_words<4>(rin, a11 == kOutOfRange ? kOutOfRange : a11 + 16u * t, q11);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float gc = gyh[4 * t + c];
              G00 = fmaf(gc, __uint_as_float(q00[c]), G00);
              G01 = fmaf(gc, __uint_as_float(q01[c]), G01);
              G10 = fmaf(gc, __uint_as_float(q10[c]), G10);
              G11 = fmaf(gc, __uint_as_float(q11[c]), G11);
            }
          }
        }
      }
      const float T = hx * G00 + lx * G01, Bt = hx * G10 + lx * G11;
      gb[k] += hy * T + ly * Bt;
      gdy[k] += Bt - T;
      gdx[k] += hy * (G01 - G00) + ly * (G11 - G10);

      // Scatter m_k * w_corner * gy_c.  In-window samples go to the LDS
      // window as scaled integers (a sample outside it adds into the sink
      // rows); the others, and every sample of a non-finite half, go to
      // grad_input with fp32 global atomics.
      // At step q lane l adds channel pair (q + l) mod 4: with 32-byte pixel
      // slices a common order would put every lane of an instruction in the
      // same few of the 64 LDS banks.  Samples outside the window add nothing
      // here (their lanes are masked off, so the sink rows see no traffic).
      if (fixed && inside) {
        const float s00 = w00 * S, s01 = w01 * S, s10 = w10 * S, s11 = w11 * S;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const float ga = gyr[2 * q], gb2 = gyr[2 * q + 1];
          unsigned char *d = gwin + A + cro[q];
          lds_iadd2(d, __float2int_rn(s00 * ga), __float2int_rn(s00 * gb2));
          lds_iadd2(d + PIXB, __float2int_rn(s01 * ga), __float2int_rn(s01 * gb2));
          lds_iadd2(d + ROW, __float2int_rn(s10 * ga), __float2int_rn(s10 * gb2));
          lds_iadd2(d + ROW + PIXB, __float2int_rn(s11 * ga), __float2int_rn(s11 * gb2));
        }
      }
      const bool gscatter = fixed ? fb : (live && !nan_loc);
      if (__builtin_amdgcn_ballot_w64(gscatter) != 0) {
        if (gscatter) {
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            const float gc = gyh[c];
            const uint32_t cb = 4u * c;
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(w00 * gc, rgx, (int)(a00 == kOutOfRange ? kOutOfRange : a00 + cb), 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(w01 * gc, rgx, (int)(a01 == kOutOfRange ? kOutOfRange : a01 + cb), 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(w10 * gc, rgx, (int)(a10 == kOutOfRange ? kOutOfRange : a10 + cb), 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(w11 * gc, rgx, (int)(a11 == kOutOfRange ? kOutOfRange : a11 + cb), 0, 0);
          }
        }
      }
    }

    __syncthreads();  // every scatter into gwin is done
    // Add the grad half-window to grad_input.  The L2 executes global
    // atomics per cache line touched, so eight consecutive lanes take one
    // pixel's 8 channels (32 contiguous bytes) and a wave covers 8 pixels;
    // pixels outside the map and zero sums are skipped.
    {
      const uint32_t c8 = lane % CH, p8 = lane / CH;
      const uint32_t cbyte = (g * CG + h * CH + c8) * 4u;
#pragma unroll 2
      for (int idx = (int)p8; idx < SPAN; idx += kBwdThreads / CH) {
        const int sy = idx / SPAN_W, sx = idx - sy * SPAN_W;
        const int gy_ = Y0 + sy, gx_ = X0 + sx;
        const bool ok = (uint32_t)gy_ < (uint32_t)p.H && (uint32_t)gx_ < (uint32_t)p.W;
        const int2 pr = unpack_pair(*reinterpret_cast<const uint64_t *>(gwin + idx * PIXB + (c8 / 2) * 8));
        const int q = (c8 & 1) ? pr.y : pr.x;
        const uint32_t dst = img + (uint32_t)gy_ * row_bytes + (uint32_t)gx_ * pix_bytes + cbyte;
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32((float)q * invS, rgx, (int)((ok && q != 0) ? dst : kOutOfRange), 0, 0);
      }
    }
  }

  if (!live) return;
  // Offset and mask gradients of the own pixel-group.  A NaN sampling
  // location makes its point's offset gradient and gm NaN.
  float2 *goff = static_cast<float2 *>(bp.grad_offset) + (uint64_t)pg * K;
  float *gmask = static_cast<float *>(bp.grad_mask) + (uint64_t)pg * K;
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float dx = s * off[2 * k], dy = s * off[2 * k + 1];
    const bool nan_loc = (dx != dx) | (dy != dy);
    if (nan_loc) gb[k] = qnan;
    goff[k] = nan_loc ? make_float2(qnan, qnan) : make_float2(s * m[k] * gdx[k], s * m[k] * gdy[k]);
  }
  if constexpr (SOFTMAX) {
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) dot = fmaf(m[k], gb[k], dot);
#pragma unroll
    for (int k = 0; k < K; ++k) gmask[k] = m[k] * (gb[k] - dot);
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) gmask[k] = gb[k];
  }
}

namespace {

template <bool SM>
hipError_t launch_bwd_tile(const BwdParams &p, const TileGeom &tg, hipStream_t s) {
  auto kern = dcn_bwd_tile_kernel<SM>;
  const size_t lds = 2 * (size_t)kBwdWinBytes + 32;  // two windows + the wave bounds
  // Set on every launch: the limit is per device and setting it is idempotent.
  const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(tg.items), dim3(kBwdThreads), lds, s, p, tg);
  return hipGetLastError();
}

}  // namespace

// 3x3 points, stride 1, dilation 1 only; hipErrorNotSupported otherwise.
hipError_t launch_backward_tiled(int softmax, const BwdParams &b, hipStream_t s) {
  const FwdParams &p = b.f;
  if (p.RC || p.KH != 3 || p.KW != 3 || p.SH != 1 || p.SW != 1 || p.DH != 1 || p.DW != 1)
    return hipErrorNotSupported;
  TileGeom tg{};
  tg.span_h = tg.span_w = kBwdSpan;
  const int tiles_y = (p.Ho + kBwdTile - 1) / kBwdTile;
  tg.tiles_x = (p.Wo + kBwdTile - 1) / kBwdTile;
  tg.tiles_per_img = tiles_y * tg.tiles_x;
  const int64_t imgs = p.pg_total / ((int64_t)p.Ho * p.Wo * p.G);
  const int64_t items = imgs * tg.tiles_per_img * p.G;
  if (items <= 0 || items >= (int64_t(1) << 31)) return hipErrorNotSupported;
  tg.items = (uint32_t)items;
  tg.div_g = make_fast_div((uint32_t)p.G);
  tg.div_tiles = make_fast_div((uint32_t)tg.tiles_per_img);
  tg.div_tiles_x = make_fast_div((uint32_t)tg.tiles_x);
  tg.div_span_w = make_fast_div((uint32_t)tg.span_w);
  return softmax ? launch_bwd_tile<true>(b, tg, s) : launch_bwd_tile<false>(b, tg, s);
}

}  // namespace dcn
