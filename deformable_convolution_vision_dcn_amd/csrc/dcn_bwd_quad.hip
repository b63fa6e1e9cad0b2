// dcn_bwd_quad.hip -- LDS-tiled gfx950 backward kernel of the DCN core
// (fp32 arithmetic for fp32 and 16-bit I/O), a lane quad per pixel-group, for
// 3x3 kernel points at stride 1 and dilation 1 (the InternImage
// configuration; wmrh.cn/news/61976, section 二 steps 2-4 and section 三) or
// 2, all nine or the eight left by DCNv4's remove_center
// (pnsm.cn/news/2029644.html section 3.3).
//
// The derivatives are those of the untiled backward kernel: every in-map
// corner of a sample receives m_k * w_corner * gy_c; the offset gradient is
// s * m_k * sum_c gy_c * dB_k[c]/d(px, py) (one-sided from the right at integer
// coordinates); the mask gradient is gm_k = sum_c gy_c * B_k[c], through the
// softmax Jacobian for DCNv3.
//
// Layout of the work: persistent 1024-thread blocks, one per CU, each walking
// (image, 16x16 output tile, group) items.  A block stages the input window
// its samples can reach (the tile's 3x3 footprint plus a halo of R pixels,
// all 16 channels of the group, 64 bytes per pixel) in LDS, and accumulates
// the grad_input scatter of the item in a second LDS window in fixed point;
// both windows fit one CU's LDS together.  At the end of the item the grad
// window is added to grad_input with global atomics, one 64-byte request per
// window pixel, and cleared for the next item.  The next item's input window,
// offset/mask rows and grad_output are requested into registers while the
// current item computes.
//
// Per pixel-group one quad: lane `sub` owns channels [4 sub, 4 sub + 4) and
// computes the location, bilinear weights (modulation folded in) and window
// address of the points k = 2 sub, 2 sub + 1 (and k = 8 for sub 0 when the
// centre is kept), as in the tiled forward.  For each point the quad reads its four corners (each lane
// its 4 channels), forms the four per-corner dot products with grad_output
// and sums them over the quad (DPP), which gives the owner the point's
// gm, d/dx and d/dy; it scatters w_corner * gy_c for its 4 channels into the
// grad window, two channels per 64-bit integer add.
// Samples whose corners leave the window take the global path behind a wave
// ballot: buffer loads for the corners and buffer atomics for the scatter.
#include <algorithm>
#include <type_traits>

#include "dcn_device.hpp"
#include "quad_ops.hpp"

namespace dcn {

#ifndef DCN_BQ_HALO
#define DCN_BQ_HALO 7
#endif
constexpr int kBqHalo = DCN_BQ_HALO;
constexpr int kBqPixB = 64;                               // 16 fp32 channels

// Block geometry for TW x TH output tiles (a quad per pixel): 16x16 (1024
// threads), 24x8 (768 threads) for maps 24 pixels wide or 12x12 (576
// threads) for 12x12 maps, both of which 16x16 tiles would leave 44 % empty.
template <int TW, int TH>
struct BqGeom {
  static constexpr int kThreads = 4 * TW * TH;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kSpanW = TW + 2 * kBqHalo + 3;     // window edges, pixels
  static constexpr int kSpanH = TH + 2 * kBqHalo + 3;
  static constexpr int kRow = kSpanW * kBqPixB;           // LDS bytes per window row
  static constexpr int kWin = kSpanW * kSpanH * kBqPixB;  // one window
  static constexpr int kZero = kRow + 2 * kBqPixB;        // zero block after the input window
  static constexpr int kSink = kRow + 2 * kBqPixB;        // scatter sink after the grad window
  static constexpr size_t kLds = (size_t)kWin + kZero + kWin + kSink + 4 * kWaves;
};

namespace {

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

}  // namespace

// RC: the centre point is removed (8 points, k -> grid index k + (k >= 4)):
// each lane owns exactly two points, lane 0's third slot stays empty and the
// item takes two rounds instead of three.
// DIL: the dilation (1 or 2, both axes).  The window keeps its size: the
// halo shrinks by one pixel per side at dilation 2.
template <int DT, bool SOFTMAX, bool RC, int DIL, int TW, int TH>
__global__ void __launch_bounds__(4 * TW * TH, (TW * TH) / 64) dcn_bwd_quad_kernel(BwdParams bp, TileGeom tg) {
  using G = BqGeom<TW, TH>;
  const FwdParams &p = bp.f;
  using io = Io<DT>;
  constexpr int EB = io::kBytes;         // bytes per element in memory
  constexpr int LB = 4 * EB;             // a lane's 4 channels in memory
  constexpr int NWL = LB / 4;            // words of them: 4 (fp32) or 2 (16-bit)
  // grad_input is accumulated in fp32 for every I/O dtype (for 16-bit I/O in
  // a caller's fp32 workspace of the input's shape): an input byte address
  // times GX is the same element's address there.
  constexpr uint32_t GX = 4 / EB;
  constexpr int R = kBqHalo - (DIL - 1), SPAN_W = G::kSpanW, SPAN_H = G::kSpanH;
  static_assert(DIL == 1 || DIL == 2, "dilation 1 or 2");
  constexpr int SPAN = SPAN_W * SPAN_H;
  constexpr int PIXB = kBqPixB, ROW = G::kRow, LIM_X = SPAN_W - 2, LIM_Y = SPAN_H - 2;
  constexpr int CG = kGroupChannels, K = RC ? 8 : 9;
  constexpr int ROUNDS = RC ? 2 : 3;
  constexpr int WPIX = G::kThreads / 4;                  // window pixels per staging slice
  constexpr int SLOTS = (SPAN + WPIX - 1) / WPIX;
  constexpr uint32_t ZERO = G::kWin;                     // zero block (reads of outside samples)
  constexpr uint32_t GWIN = G::kWin + G::kZero;          // fixed-point grad window
  constexpr uint32_t SINK = GWIN + G::kWin;              // scatter target of samples not in the window
  static_assert(CG == 16, "a quad covers 16 channels");

  extern __shared__ __align__(16) unsigned char lds[];
  typedef __attribute__((address_space(3))) unsigned char lds_byte;
  const uint32_t lbase = (uint32_t)(size_t)(lds_byte *)lds;
  float *wave_sums = reinterpret_cast<float *>(lds + SINK + G::kSink);

  const uint32_t quad = threadIdx.x >> 2, sub = threadIdx.x & 3;
  const int oy = (int)quad / TW, ox = (int)quad % TW;  // output pixel within the tile
  const uint32_t pix_bytes = (uint32_t)p.C * EB;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const __amdgpu_buffer_rsrc_t rgx = make_rsrc(bp.grad_in, p.in_bytes * GX);
  const __amdgpu_buffer_rsrc_t roff = make_rsrc(p.offset, p.off_bytes);
  const __amdgpu_buffer_rsrc_t rmask = make_rsrc(p.mask, p.mask_bytes);
  const __amdgpu_buffer_rsrc_t rgy = make_rsrc(bp.grad_out, p.pg_total * (uint32_t)(CG * EB));
  const __amdgpu_buffer_rsrc_t rgoff = make_rsrc(bp.grad_offset, p.off_bytes);
  const __amdgpu_buffer_rsrc_t rgm = make_rsrc(bp.grad_mask, p.mask_bytes);
  const float s = p.scale;

  // Window coordinates of each own slot's kernel point before its offset,
  // packed as three 10-bit fields; slot r holds k = 2 sub + r (r < 2) or 8
  // (no point with RC), at grid index q.
  uint32_t bxp = 0, byp = 0;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int k = r < 2 ? 2 * (int)sub + r : 8;
    const int q = RC ? (r < 2 ? k + (k >= 4) : 4) : k;
    bxp |= (uint32_t)(ox + R + (q % 3) * DIL) << (10 * r);
    byp |= (uint32_t)(oy + R + (q / 3) * DIL) << (10 * r);
  }
  const uint32_t win_chunk = lbase + sub * 16u;          // this lane's 4 channels of a window pixel
  const uint32_t gwin_chunk = lbase + GWIN + sub * 16u;

  // The grad window starts at zero; every item's flush clears it again.  The
  // zero block after the input window is written once.  The first barrier of
  // the item loop orders both.
  for (uint32_t z = threadIdx.x * 16u; z < (uint32_t)G::kWin; z += G::kThreads * 16u)
    *reinterpret_cast<uint4 *>(lds + GWIN + z) = make_uint4(0, 0, 0, 0);
  for (uint32_t z = threadIdx.x * 16u; z < (uint32_t)G::kZero; z += G::kThreads * 16u)
    *reinterpret_cast<uint4 *>(lds + ZERO + z) = make_uint4(0, 0, 0, 0);

  struct Item {
    uint32_t g, n, img, chan, pg;
    int Y0, X0;
    bool live;
  };
  auto decode = [&](uint32_t it) {
    Item I;
    const uint32_t t = fast_div(it, tg.div_g);
    I.g = it - t * (uint32_t)p.G;
    I.n = fast_div(t, tg.div_tiles);
    const uint32_t tile_id = t - I.n * (uint32_t)tg.tiles_per_img;
    const uint32_t tyi = fast_div(tile_id, tg.div_tiles_x);
    const uint32_t txi = tile_id - tyi * (uint32_t)tg.tiles_x;
    const int r0 = (int)tyi * TH, c0 = (int)txi * TW;
    I.Y0 = r0 - p.PH - R;  // window origin in input coordinates
    I.X0 = c0 - p.PW - R;
    I.img = I.n * (uint32_t)p.H * row_bytes;
    I.chan = I.g * (uint32_t)(CG * EB) + sub * (uint32_t)LB;
    const int ho = r0 + oy, wo = c0 + ox;
    I.live = ho < p.Ho && wo < p.Wo;
    I.pg = I.live ? (((I.n * (uint32_t)p.Ho + ho) * (uint32_t)p.Wo + wo) * (uint32_t)p.G) + I.g : 0u;
    return I;
  };

  // Next item's input window (4 lanes of 16 bytes per pixel), offset and mask
  // rows and grad_output: requested into registers while the current item
  // computes, on every path (a missing item loads nothing: its offsets are
  // out of range), so the compiler's count of outstanding loads stays exact.
  uint32_t win[SLOTS][NWL];
  auto issue_window = [&](const Item &I, bool valid) {
    // The slot geometry is recomputed per item from an opaque copy of the
    // quad index: hoisted out of the item loop it would not fit the
    // register budget.
    uint32_t qd = quad;
    asm volatile("" : "+v"(qd));
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const int idx = (int)qd + u * WPIX;
      uint32_t offb = kOutOfRange;
      if (valid && idx < SPAN) {
        const int sy = idx / SPAN_W, sx = idx - sy * SPAN_W;
        const int gy_ = I.Y0 + sy, gx_ = I.X0 + sx;
        if ((uint32_t)gy_ < (uint32_t)p.H && (uint32_t)gx_ < (uint32_t)p.W)
          offb = I.img + (uint32_t)gy_ * row_bytes + (uint32_t)gx_ * pix_bytes + I.chan;
      }
      buffer_load_words<NWL>(rin, offb, win[u]);
    }
  };
  auto store_window = [&]() {
    uint32_t qd = quad;
    asm volatile("" : "+v"(qd));
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const int idx = (int)qd + u * WPIX;
      if (idx < SPAN) {  // staged as fp32 whatever the I/O dtype
        float v[4];
        unpack<DT, NWL>(win[u], v);
        *reinterpret_cast<uint4 *>(lds + idx * PIXB + sub * 16u) =
            make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
      }
    }
  };
  // Raw rows as loaded (decoded where used).  fp32: rw = x, y of k = 2 sub;
  // x, y of 2 sub + 1; x, y of 8; rl = logits of 2 sub, 2 sub + 1, 8; rg =
  // grad_output of the lane's 4 channels.  16-bit: rw = (x, y) words of
  // 2 sub, 2 sub + 1, 8; rl = the three logits (low halves); rg = two words.
  constexpr int NRW = DT == DCN_F32 ? 6 : 3;
  uint32_t rw[NRW], rl[3], rg[NWL];
  auto issue_rows = [&](const Item &I) {
    if constexpr (DT == DCN_F32) {
      const uint32_t orow = I.pg * (K * 8), mrow = I.pg * (K * 4);
      const auto o = __builtin_amdgcn_raw_buffer_load_b128(roff, (int)(orow + 16 * sub), 0, 0);
      const auto lg = __builtin_amdgcn_raw_buffer_load_b64(rmask, (int)(mrow + 8 * sub), 0, 0);
      if constexpr (RC) {
        rw[4] = rw[5] = rl[2] = 0u;
      } else {
        const auto o8 = __builtin_amdgcn_raw_buffer_load_b64(roff, (int)(orow + 64), 0, 0);
        rl[2] = __builtin_amdgcn_raw_buffer_load_b32(rmask, (int)(mrow + 32), 0, 0);
        rw[4] = o8[0];
        rw[5] = o8[1];
      }
      rw[0] = o[0];
      rw[1] = o[1];
      rw[2] = o[2];
      rw[3] = o[3];
      rl[0] = lg[0];
      rl[1] = lg[1];
    } else {
      const uint32_t orow = I.pg * (K * 4), mrow = I.pg * (K * 2);
      const auto o = __builtin_amdgcn_raw_buffer_load_b64(roff, (int)(orow + 8 * sub), 0, 0);
      rw[0] = o[0];
      rw[1] = o[1];
      if constexpr (RC) {  // 16-byte mask rows: the lane's two logits in one word
        const uint32_t lw = __builtin_amdgcn_raw_buffer_load_b32(rmask, (int)(mrow + 4 * sub), 0, 0);
        rl[0] = lw & 0xffffu;
        rl[1] = lw >> 16;
        rw[2] = rl[2] = 0u;
      } else {
        rw[2] = __builtin_amdgcn_raw_buffer_load_b32(roff, (int)(orow + 32), 0, 0);
        rl[0] = __builtin_amdgcn_raw_buffer_load_b16(rmask, (int)(mrow + 4 * sub), 0, 0);
        rl[1] = __builtin_amdgcn_raw_buffer_load_b16(rmask, (int)(mrow + 4 * sub + 2), 0, 0);
        rl[2] = __builtin_amdgcn_raw_buffer_load_b16(rmask, (int)(mrow + 16), 0, 0);
      }
    }
    buffer_load_words<NWL>(rgy, I.pg * (uint32_t)(CG * EB) + sub * (uint32_t)LB, rg);
  };

  const XcdWalk walk = xcd_walk(blockIdx.x, gridDim.x, tg.items);
  const uint32_t end = walk.end;
  uint32_t item = walk.first;
  Item cur = decode(item < end ? item : 0);
  if (item < end) {
    issue_window(cur, true);
    issue_rows(cur);
  }
  const float qnan = __builtin_nanf("");

  while (item < end) {
    __syncthreads();  // the previous item's reads, scatters and flush are done
    store_window();

    // Own slots: offsets, modulation weights (softmax over the quad's nine
    // logits for DCNv3, the raw mask for DCNv4) and grad_output.
    float2 offs[3];
    float m[3], gy[4];
    float lgs[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      if constexpr (DT == DCN_F32)
        offs[r] = make_float2(__uint_as_float(rw[2 * r]), __uint_as_float(rw[2 * r + 1]));
      else
        offs[r] = make_float2(io::lo(rw[r]), io::hi(rw[r]));
      lgs[r] = io::lo(rl[r]);
    }
    unpack<DT, NWL>(rg, gy);
    if (RC || sub != 0) lgs[2] = SOFTMAX ? -INFINITY : 0.f;  // slot 2 is lane 0's point 8 only
    if constexpr (SOFTMAX) {
      const float mx = quad_max(fmaxf(fmaxf(lgs[0], lgs[1]), lgs[2]));
      float e[3], sum = 0.f;
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        e[r] = (r < 2 || (!RC && sub == 0)) ? __expf(lgs[r] - mx) : 0.f;
        sum += e[r];
      }
      const float inv = __builtin_amdgcn_rcpf(quad_sum(sum));
#pragma unroll
      for (int r = 0; r < 3; ++r) m[r] = e[r] * inv;
    } else {
#pragma unroll
      for (int r = 0; r < 3; ++r) m[r] = lgs[r];
    }

    // Fixed-point scale of the item's grad window.  Every window
    // pixel-channel receives at most the sum over the tile's pixel-groups of
    // sum_k |m_k| * max_c |gy_c| (the four corner weights of a sample are
    // non-negative and add up to 1), call it B.  With S = 2^(30 - e), B <= 2^e,
    // every partial sum of the scaled terms stays within 2^30, so the LDS
    // integer adds sum them exactly; each term is rounded to the nearest
    // multiple of 1/S.  A non-finite B (NaN or Inf in grad_output or the mask)
    // sends the whole item to fp32 global atomics instead.
    {
      float gmax = 0.f, nanflag = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        gmax = fmaxf(gmax, fabsf(gy[c]));
        nanflag += 0.f * gy[c];  // fmaxf drops NaN: a NaN in gy must still reach the bound
      }
      const float msum = quad_sum(fabsf(m[0]) + fabsf(m[1]) + fabsf(m[2]));
      float bound = quad_max(gmax) * msum + quad_sum(nanflag);
      bound = (cur.live && sub == 0) ? bound : 0.f;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) bound += __shfl_xor(bound, d, 64);
      if ((threadIdx.x & 63) == 0) wave_sums[threadIdx.x >> 6] = bound;
    }
    __syncthreads();  // the window is in LDS, the wave bounds are ready

    float B = 0.f;
#pragma unroll
    for (int wv = 0; wv < G::kWaves; ++wv) B += wave_sums[wv];
    const bool fixed = B <= 3.0e38f;  // false for Inf and NaN (block-uniform)
    int ex = 0;
    frexpf(B, &ex);
    ex = ex < -96 ? -96 : ex;
    const float S = ldexpf(1.f, 30 - ex), invS = ldexpf(1.f, ex - 30);

    const uint32_t next = item + walk.stride;
    const bool more = next < end;  // block-uniform
    const Item nx = decode(more ? next : item);
    issue_window(nx, more);
    issue_rows(nx);

    // Per-slot results, shifted in round by round: after the three rounds
    // (two with RC, then one empty shift) res2 holds slot 0, res1 slot 1,
    // res0 slot 2.  (gm, d/dx, d/dy)
    float3 res0 = make_float3(0.f, 0.f, 0.f), res1 = res0, res2 = res0;
    float2 o2 = offs[0], o2n = offs[1], o2nn = offs[2];
    float mk = m[0], mkn = m[1], mknn = m[2];
#pragma unroll 1
    for (int r = 0; r < ROUNDS; ++r) {
      // Wave priority falls round by round: the waves furthest behind issue
      // first, so the block reaches its flush barrier with less spread.
      if (r == 0) __builtin_amdgcn_s_setprio(3);
      if (r == 1) __builtin_amdgcn_s_setprio(2);
      if (r == 2) __builtin_amdgcn_s_setprio(1);
      const float dx = s * o2.x, dy = s * o2.y;
      const bool nan_loc = (dx != dx) | (dy != dy);
      const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
      const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
      const float fx = floorf(cx), fy = floorf(cy);
      const float lx = cx - fx, ly = cy - fy;
      const float hx = 1.f - lx, hy = 1.f - ly;
      const int tx = (int)((bxp >> (10 * r)) & 1023u) + (int)fx;  // window coordinates
      const int ty = (int)((byp >> (10 * r)) & 1023u) + (int)fy;
      const bool inside = cur.live && !nan_loc && (uint32_t)ty <= (uint32_t)LIM_Y && (uint32_t)tx <= (uint32_t)LIM_X;
      const uint32_t A = inside ? mad24((uint32_t)ty, (uint32_t)ROW, mul24((uint32_t)tx, PIXB)) : ZERO;
      const float wy1 = ly * mk, wy0 = mk - wy1;
      const float W1 = wy0 * lx, W0 = wy0 - W1;
      const float W3 = wy1 * lx, W2 = wy1 - W3;
      // scaled to the fixed-point grid for the LDS scatter
      const float W0s = W0 * S, W1s = W1 * S, W2s = W2 * S, W3s = W3 * S;
      // outside the window but touching the map: global gathers and atomics
      const bool fb = cur.live && !inside && !nan_loc && (uint32_t)(cur.Y0 + 1 + ty) <= (uint32_t)p.H &&
                      (uint32_t)(cur.X0 + 1 + tx) <= (uint32_t)p.W;
      // LDS scatter target: the window, or the sink for samples it does not
      // hold (outside it, NaN locations, dead lanes), which is never read.
      const uint32_t AS = inside ? A : SINK - GWIN;
      const bool gscat = fixed ? fb : (cur.live && !nan_loc);  // global scatter
      const bool fb_any = __builtin_amdgcn_ballot_w64(fb) != 0;      // wave-uniform
      const bool gs_any = __builtin_amdgcn_ballot_w64(gscat) != 0;   // wave-uniform
      float3 mine = make_float3(0.f, 0.f, 0.f);

      auto point = [&](auto o_tag) {
        constexpr int O = decltype(o_tag)::value;
        // Gather this lane's 4 channels of the owner's four corners.
        const uint32_t src = add_bcast<O>(A, win_chunk);
        uint32_t q00[4], q01[4], q10[4], q11[4];
        lds_load_at<4>(src, q00);
        lds_load_at<4>(src + PIXB, q01);
        lds_load_at<4>(src + ROW, q10);
        lds_load_at<4>(src + ROW + PIXB, q11);
        float P[4] = {0.f, 0.f, 0.f, 0.f};  // corners 00, 01, 10, 11
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          P[0] = fmaf(gy[c], __uint_as_float(q00[c]), P[0]);
          P[1] = fmaf(gy[c], __uint_as_float(q01[c]), P[1]);
          P[2] = fmaf(gy[c], __uint_as_float(q10[c]), P[2]);
          P[3] = fmaf(gy[c], __uint_as_float(q11[c]), P[3]);
        }
        // Global byte offsets of the owner's four corners for this lane's
        // channels (out of range where a corner is outside the map).
        auto corners = [&](uint32_t (&ga)[4]) {
          const int yb = qbcast<O>(ty) + cur.Y0, xb = qbcast<O>(tx) + cur.X0;
          const bool vy0 = (uint32_t)yb < (uint32_t)p.H, vy1 = (uint32_t)(yb + 1) < (uint32_t)p.H;
          const bool vx0 = (uint32_t)xb < (uint32_t)p.W, vx1 = (uint32_t)(xb + 1) < (uint32_t)p.W;
          const uint32_t a00 = cur.img + (uint32_t)yb * row_bytes + (uint32_t)xb * pix_bytes + cur.chan;
          ga[0] = (vy0 && vx0) ? a00 : kOutOfRange;
          ga[1] = (vy0 && vx1) ? a00 + pix_bytes : kOutOfRange;
          ga[2] = (vy1 && vx0) ? a00 + row_bytes : kOutOfRange;
          ga[3] = (vy1 && vx1) ? a00 + row_bytes + pix_bytes : kOutOfRange;
        };
        if (fb_any) {  // a quad of the wave left its window this round
          if (qbcast<O>((int)fb)) {
            uint32_t ga[4];
            corners(ga);
            uint32_t r00[NWL], r01[NWL], r10[NWL], r11[NWL];
            buffer_load_words<NWL>(rin, ga[0], r00);
            buffer_load_words<NWL>(rin, ga[1], r01);
            buffer_load_words<NWL>(rin, ga[2], r10);
            buffer_load_words<NWL>(rin, ga[3], r11);
            float v00[4], v01[4], v10[4], v11[4];
            unpack<DT, NWL>(r00, v00);
            unpack<DT, NWL>(r01, v01);
            unpack<DT, NWL>(r10, v10);
            unpack<DT, NWL>(r11, v11);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              P[0] = fmaf(gy[c], v00[c], P[0]);
              P[1] = fmaf(gy[c], v01[c], P[1]);
              P[2] = fmaf(gy[c], v10[c], P[2]);
              P[3] = fmaf(gy[c], v11[c], P[3]);
            }
          }
        }
        // Sums over the 16 channels: every lane of the quad gets them; the
        // owner keeps gm, d/dx and d/dy of its point (one-sided derivatives
        // of the bilinear form, linear in the corner sums).
        quad_sum4(P);
        const float G00 = P[0], G01 = P[1], G10 = P[2], G11 = P[3];
        if (sub == (uint32_t)O) {
          const float T = hx * G00 + lx * G01, Bt = hx * G10 + lx * G11;
          mine = nan_loc ? make_float3(qnan, qnan, qnan)
                         : make_float3(hy * T + ly * Bt, hy * (G01 - G00) + ly * (G11 - G10), Bt - T);
        }
        // Scatter m_k * w_corner * gy_c of this lane's 4 channels (no
        // branch: samples the window does not hold add into the sink).
        if (fixed) {  // block-uniform
          const uint32_t d = add_bcast<O>(AS, gwin_chunk);
          auto corner = [&](float w, uint32_t at) {
            float t[4];
            mul4_bcast<O>(t, w, gy);
            lds_add_pair(at, cvt_rpi(t[0]), cvt_rpi(t[1]));
            lds_add_pair(at + 8, cvt_rpi(t[2]), cvt_rpi(t[3]));
          };
          corner(W0s, d);
          corner(W1s, d + PIXB);
          corner(W2s, d + ROW);
          corner(W3s, d + ROW + PIXB);
        }
        if (gs_any) {
          if (qbcast<O>((int)gscat)) {
            uint32_t ga[4];
            corners(ga);
            const float wc[4] = {qbcast<O>(W0), qbcast<O>(W1), qbcast<O>(W2), qbcast<O>(W3)};
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int c = 0; c < 4; ++c)
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                    wc[q] * gy[c], rgx, (int)(ga[q] == kOutOfRange ? kOutOfRange : ga[q] * GX + 4u * c), 0, 0);
          }
        }
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      point(I0{});
      if (r < 2) {  // the last round holds only k = 8 (owner lane 0)
        point(I1{});
        point(I2{});
        point(I3{});
      }
      res2 = res1;
      res1 = res0;
      res0 = mine;
      o2 = o2n;
      o2n = o2nn;
      mk = mkn;
      mkn = mknn;
    }

    if constexpr (RC) {
      res2 = res1;
      res1 = res0;
      res0 = make_float3(0.f, 0.f, 0.f);
    }

    // Offset and mask gradients of the own slots (a NaN sampling location
    // makes its point's offset gradient and gm NaN).
    if (cur.live) {
      const float3 rs[3] = {res2, res1, res0};
      float gm[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) gm[r] = rs[r].x;
      if constexpr (SOFTMAX) {
        float dot = m[0] * gm[0] + m[1] * gm[1];
        if (!RC && sub == 0) dot += m[2] * gm[2];
        dot = quad_sum(dot);
#pragma unroll
        for (int r = 0; r < 3; ++r) gm[r] = m[r] * (gm[r] - dot);
      }
      // offset gradients (x, y) of the three slots
      float go[3][2];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        go[r][0] = s * m[r] * rs[r].y;
        go[r][1] = s * m[r] * rs[r].z;
      }
      if constexpr (DT == DCN_F32) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        const uint32_t orow = cur.pg * (K * 8), mrow = cur.pg * (K * 4);
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(4))), f4{go[0][0], go[0][1], go[1][0], go[1][1]}),
            rgoff, (int)(orow + 16 * sub), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))), f2{gm[0], gm[1]}), rgm,
            (int)(mrow + 8 * sub), 0, 0);
        if (!RC && sub == 0) {
          __builtin_amdgcn_raw_buffer_store_b64(
              __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))), f2{go[2][0], go[2][1]}), rgoff,
              (int)(orow + 64), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gm[2]), rgm, (int)(mrow + 32), 0, 0);
        }
      } else {  // rounded to the I/O dtype; the 18-byte mask rows take 2-byte stores
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const uint32_t orow = cur.pg * (K * 4), mrow = cur.pg * (K * 2);
        __builtin_amdgcn_raw_buffer_store_b64(u2{io::pack(go[0][0], go[0][1]), io::pack(go[1][0], go[1][1])}, rgoff,
                                              (int)(orow + 8 * sub), 0, 0);
        const uint32_t gmw = io::pack(gm[0], gm[1]);
        if constexpr (RC) {  // 16-byte mask rows: one aligned word per lane
          __builtin_amdgcn_raw_buffer_store_b32(gmw, rgm, (int)(mrow + 4 * sub), 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(gmw & 0xffffu), rgm, (int)(mrow + 4 * sub), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(gmw >> 16), rgm, (int)(mrow + 4 * sub + 2), 0, 0);
        }
        if (!RC && sub == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(io::pack(go[2][0], go[2][1]), rgoff, (int)(orow + 32), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(io::pack(gm[2], 0.f) & 0xffffu), rgm,
                                                (int)(mrow + 16), 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_setprio(0);
    __syncthreads();  // every scatter into the grad window is done
    // Add the grad window to grad_input, 16 lanes per window pixel (one
    // 64-byte request), and clear it for the next item.  Pixels outside the
    // map and zero sums are skipped.
    {
      // Pixel idx = threadIdx.x / 16 + STEP j of the window, its row, column
      // and grad_input offset walked incrementally.
      constexpr int STEP = G::kThreads / 16;
      constexpr int DY = STEP / SPAN_W, DX = STEP % SPAN_W;
      const uint32_t ch = threadIdx.x & 15u;
      int idx = (int)(threadIdx.x >> 4);
      int sy = idx / SPAN_W, sx = idx - sy * SPAN_W;
      uint32_t dst = cur.img + (uint32_t)(cur.Y0 + sy) * row_bytes + (uint32_t)(cur.X0 + sx) * pix_bytes +
                     cur.g * (uint32_t)(CG * EB) + ch * (uint32_t)EB;
      const uint32_t slot0 = lbase + GWIN + (ch >> 1) * 8u;
      typedef __attribute__((address_space(3))) uint64_t L;
#pragma unroll 2
      for (; idx < SPAN; idx += STEP) {
        const bool ok = (uint32_t)(cur.Y0 + sy) < (uint32_t)p.H && (uint32_t)(cur.X0 + sx) < (uint32_t)p.W;
        L *slot = (L *)(size_t)(slot0 + (uint32_t)idx * PIXB);
        const int2 pr = pair_sums(*slot);
        if ((ch & 1u) == 0) *slot = 0;  // after both lanes of the pair have read it (same instruction)
        const int q = (ch & 1u) ? pr.y : pr.x;
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32((float)q * invS, rgx, (int)((ok && q != 0) ? dst * GX : kOutOfRange), 0, 0);
        sx += DX;
        sy += DY;
        dst += (uint32_t)DY * row_bytes + (uint32_t)DX * pix_bytes;
        if (sx >= SPAN_W) {
          sx -= SPAN_W;
          sy += 1;
          dst += row_bytes - (uint32_t)SPAN_W * pix_bytes;
        }
      }
    }

    item = next;
    cur = nx;
  }
}

namespace {

template <int DT, bool SM, bool RC, int DIL, int TW, int TH>
hipError_t launch_bwd_quad(const BwdParams &p, const TileGeom &tg, hipStream_t s) {
  using G = BqGeom<TW, TH>;
  auto kern = dcn_bwd_quad_kernel<DT, SM, RC, DIL, TW, TH>;
  // Set on every launch: the limit is per device and setting it is idempotent.
  const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::kLds);
  if (attr != hipSuccess) return attr;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), G::kThreads,
                                                     G::kLds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorNotSupported;
  const uint32_t blocks = std::min<uint32_t>(tg.items, (uint32_t)per_cu * (uint32_t)cus);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(G::kThreads), G::kLds, s, p, tg);
  return hipGetLastError();
}

template <bool RC, int DIL, int TW, int TH>
hipError_t launch_dt(int dtype, int softmax, const BwdParams &b, const TileGeom &tg, hipStream_t s) {
  switch (dtype) {
    case DCN_F32:
      return softmax ? launch_bwd_quad<DCN_F32, true, RC, DIL, TW, TH>(b, tg, s)
                     : launch_bwd_quad<DCN_F32, false, RC, DIL, TW, TH>(b, tg, s);
    case DCN_F16:
      return softmax ? launch_bwd_quad<DCN_F16, true, RC, DIL, TW, TH>(b, tg, s)
                     : launch_bwd_quad<DCN_F16, false, RC, DIL, TW, TH>(b, tg, s);
    case DCN_BF16:
      return softmax ? launch_bwd_quad<DCN_BF16, true, RC, DIL, TW, TH>(b, tg, s)
                     : launch_bwd_quad<DCN_BF16, false, RC, DIL, TW, TH>(b, tg, s);
    default: return hipErrorInvalidValue;
  }
}

// Share of the tiles' pixels that are output pixels.
double quad_tile_use(const FwdParams &p, int tw, int th) {
  const double tiled = (double)((p.Ho + th - 1) / th) * th * (double)((p.Wo + tw - 1) / tw) * tw;
  return (double)p.Ho * p.Wo / tiled;
}

}  // namespace

// 3x3 points (all nine, or eight without the centre), stride 1, dilation 1
// or 2 (the same on both axes) only; hipErrorNotSupported otherwise.
hipError_t launch_backward_quad(int dtype, int softmax, const BwdParams &b, hipStream_t s) {
  const FwdParams &p = b.f;
  if (p.KH != 3 || p.KW != 3 || p.SH != 1 || p.SW != 1 || p.DH != p.DW || (p.DH != 1 && p.DH != 2))
    return hipErrorNotSupported;
  // 24x8 or 12x12 tiles (dilation 1) where they leave clearly fewer quads
  // idle than 16x16 ones (24x8 on a tie between the two)
  const double u16 = quad_tile_use(p, 16, 16), u24 = quad_tile_use(p, 24, 8), u12 = quad_tile_use(p, 12, 12);
  const bool wide = p.DH == 1 && u24 > u16 + 0.1 && u24 >= u12;
  const bool small = p.DH == 1 && !wide && u12 > u16 + 0.1;
  const int tw = wide ? 24 : (small ? 12 : 16), th = wide ? 8 : (small ? 12 : 16);
  TileGeom tg{};
  tg.span_w = tw + 2 * kBqHalo + 3;
  tg.span_h = th + 2 * kBqHalo + 3;
  const int tiles_y = (p.Ho + th - 1) / th;
  tg.tiles_x = (p.Wo + tw - 1) / tw;
  tg.tiles_per_img = tiles_y * tg.tiles_x;
  const int64_t imgs = p.pg_total / ((int64_t)p.Ho * p.Wo * p.G);
  const int64_t items = imgs * tg.tiles_per_img * p.G;
  if (items <= 0 || items >= (int64_t(1) << 31)) return hipErrorNotSupported;
  tg.items = (uint32_t)items;
  tg.div_g = make_fast_div((uint32_t)p.G);
  tg.div_tiles = make_fast_div((uint32_t)tg.tiles_per_img);
  tg.div_tiles_x = make_fast_div((uint32_t)tg.tiles_x);
  tg.div_span_w = make_fast_div((uint32_t)tg.span_w);
  if (p.DH == 2)
    return p.RC ? launch_dt<true, 2, 16, 16>(dtype, softmax, b, tg, s) : launch_dt<false, 2, 16, 16>(dtype, softmax, b, tg, s);
  if (wide)
    return p.RC ? launch_dt<true, 1, 24, 8>(dtype, softmax, b, tg, s) : launch_dt<false, 1, 24, 8>(dtype, softmax, b, tg, s);
  if (small)
    return p.RC ? launch_dt<true, 1, 12, 12>(dtype, softmax, b, tg, s) : launch_dt<false, 1, 12, 12>(dtype, softmax, b, tg, s);
  return p.RC ? launch_dt<true, 1, 16, 16>(dtype, softmax, b, tg, s) : launch_dt<false, 1, 16, 16>(dtype, softmax, b, tg, s);
}

}  // namespace dcn
