// dcn_bwd_quad.hip -- LDS-tiled gfx950 backward kernel of the DCN core
// (fp32 arithmetic for fp32 and 16-bit I/O), a lane quad per pixel-group, for
// 3x3 kernel points at stride 1 and dilation 1 (the InternImage
// configuration; wmrh.cn/news/61976, section 二 steps 2-4 and section 三) or
// 2, also at stride 2 (the DCNv4 signature carries stride and dilation), all
// nine or the eight left by DCNv4's remove_center (pnsm.cn/news/2029644.html
// section 3.3).
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
#include "bwd_fixed.hpp"
#include "quad_ops.hpp"

namespace dcn {

#ifndef DCN_BQ_HALO
#define DCN_BQ_HALO 7
#endif
constexpr int kBqHalo = DCN_BQ_HALO;
constexpr int kBqPixB = 64;                               // 16 fp32 channels

// Halo at stride 2 (dilation 1; one less at dilation 2, so the window keeps
// its size).
constexpr int kBqHaloS2 = 4;
// Halo of 5x5 points (stride and dilation 1): a 16x16 tile's window is then
// 33 pixels on a side, as with 3x3 points and halo 7.
constexpr int kBqHalo5 = 6;

// Block geometry for TW x TH output tiles (a quad per pixel) at stride ST:
// 16x16 (1024 threads), 24x8 (768 threads) for maps 24 pixels wide or 12x12
// (576 threads) for 12x12 maps, both of which 16x16 tiles would leave 44 %
// empty; at stride 2, 16x8 tiles (512 threads) whose 42 x 26 windows (the
// footprint plus a halo of 4) fit beside their grad windows; with 5x5 points,
// 16x16 or 16x8 tiles with a halo of 6 (33 x 33 or 33 x 25 windows).
template <int TW, int TH, int ST = 1, int KS = 3>
struct BqGeom {
  static_assert(ST == 1 || ST == 2, "stride 1 or 2");
  static_assert(KS == 3 || (KS == 5 && ST == 1), "3x3 points, or 5x5 at stride 1");
  static constexpr int kHalo1 = KS == 5 ? kBqHalo5 : kBqHalo;  // stride 1, dilation 1
  static constexpr int kThreads = 4 * TW * TH;
  static constexpr int kWaves = kThreads / 64;
  // window edges, pixels: (T - 1) * ST + 2 * DIL + 2 * R + 2 with the halo R
  // one smaller at dilation 2, so independent of the dilation
  static constexpr int kSpanW = ST == 1 ? TW + 2 * kHalo1 + KS : 2 * TW + 2 * kBqHaloS2 + 2;
  static constexpr int kSpanH = ST == 1 ? TH + 2 * kHalo1 + KS : 2 * TH + 2 * kBqHaloS2 + 2;
  static constexpr int kRow = kSpanW * kBqPixB;           // LDS bytes per window row
  static constexpr int kWin = kSpanW * kSpanH * kBqPixB;  // one window
  static constexpr int kZero = kRow + 2 * kBqPixB;        // zero block after the input window
  static constexpr int kSink = kRow + 2 * kBqPixB;        // scatter sink after the grad window
  static constexpr size_t kLds = (size_t)kWin + kZero + kWin + kSink + 8 * kWaves;
};

// RC: the centre point is removed (8 points, k -> grid index k + (k >= 4)):
// each lane owns exactly two points, lane 0's third slot stays empty and the
// item takes two rounds instead of three.
// DIL: the dilation (1 or 2, both axes).  The window keeps its size: the
// halo shrinks by one pixel per side at dilation 2.
template <int DT, bool SOFTMAX, bool RC, int DIL, int TW, int TH, int ST, int KS>
__global__ void __launch_bounds__(4 * TW * TH, (TW * TH) / 64) dcn_bwd_quad_kernel(BwdParams bp, TileGeom tg) {
  using G = BqGeom<TW, TH, ST, KS>;
  const FwdParams &p = bp.f;
  using io = Io<DT>;
  constexpr int EB = io::kBytes;         // bytes per element in memory
  constexpr int LB = 4 * EB;             // a lane's 4 channels in memory
  constexpr int NWL = LB / 4;            // words of them: 4 (fp32) or 2 (16-bit)
  // grad_input is accumulated in fp32 for every I/O dtype (for 16-bit I/O in
  // a caller's fp32 workspace of the input's shape): an input byte address
  // times GX is the same element's address there.
  constexpr uint32_t GX = 4 / EB;
  constexpr int R = (ST == 1 ? G::kHalo1 : kBqHaloS2) - (DIL - 1), SPAN_W = G::kSpanW, SPAN_H = G::kSpanH;
  static_assert(DIL == 1 || DIL == 2, "dilation 1 or 2");
  constexpr int PIXB = kBqPixB, ROW = G::kRow, LIM_X = SPAN_W - 2, LIM_Y = SPAN_H - 2;
  constexpr int CG = kGroupChannels, K = KS * KS - (RC ? 1 : 0);
  // Points per lane.  3x3: lane sub owns k = 2 sub, 2 sub + 1 and (lane 0)
  // k = 8; 5x5: lane sub owns k = P sub + r, r < P, where below K.
  constexpr int P = KS == 3 ? 3 : (K + 3) / 4;
  constexpr int ROUNDS = KS == 3 ? (RC ? 2 : 3) : P;
  static_assert(KS == 3 || (DIL == 1 && ST == 1), "5x5 points at stride and dilation 1");
  constexpr int WPIX = G::kThreads / 4;                  // window pixels per staging slice
  using WS = Slices<SPAN_W, SPAN_H, WPIX>;               // input window: a quad per pixel
  using FS = Slices<SPAN_W, SPAN_H, G::kThreads / 16>;   // flush: 16 lanes per pixel
  constexpr int SLOTS = WS::N;
  constexpr uint32_t ZERO = G::kWin;                     // zero block (reads of outside samples)
  constexpr uint32_t GWIN = G::kWin + G::kZero;          // fixed-point grad window
  constexpr uint32_t SINK = GWIN + G::kWin;              // scatter target of samples not in the window
  static_assert(CG == 16, "a quad covers 16 channels");

  extern __shared__ __align__(16) unsigned char lds[];
  typedef __attribute__((address_space(3))) unsigned char lds_byte;
  const uint32_t lbase = (uint32_t)(size_t)(lds_byte *)lds;
  float *wave_sums = reinterpret_cast<float *>(lds + SINK + G::kSink);
  float *wave_mins = wave_sums + G::kWaves;

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
  const uint32_t img_bytes = (uint32_t)p.H * row_bytes;

  // This quad's input-window slices (main: row w_row + u RPS, column w_col).
  const uint32_t w_col = quad % (uint32_t)WS::CW, w_row = quad / (uint32_t)WS::CW;
  const uint32_t w_lane = w_row * row_bytes + w_col * pix_bytes;
  const uint32_t w_lds = (w_row * SPAN_W + w_col) * PIXB + sub * 16u;

  // Window coordinates of each own slot's kernel point before its offset,
  // packed as three 10-bit fields; slot r holds k = 2 sub + r (r < 2) or 8
  // (no point with RC), at grid index q.
  uint32_t bxp = 0, byp = 0;
  if constexpr (KS == 3) {
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int k = r < 2 ? 2 * (int)sub + r : 8;
      const int q = RC ? (r < 2 ? k + (k >= 4) : 4) : k;
      bxp |= (uint32_t)(ox * ST + R + (q % 3) * DIL) << (10 * r);
      byp |= (uint32_t)(oy * ST + R + (q / 3) * DIL) << (10 * r);
    }
  }
  const uint32_t win_chunk = lbase + sub * 16u;          // this lane's 4 channels of a window pixel
  // The scatter's first 64-bit add of a corner takes the lane's first channel
  // pair in even quads and its second pair in odd ones, so the four quads of
  // a 16-lane group spread over twice as many LDS banks (the layout is the
  // same: pair 0 at +0, pair 1 at +8 of the lane's 16 bytes).  Not for fp32
  // at stride 2, where it measured slower.
  constexpr bool ALT = !(DT == DCN_F32 && ST == 2);
  const uint32_t podd = ALT ? (quad & 1u) : 0u;
  const uint32_t gwin_chunk = lbase + GWIN + sub * 16u + 8u * podd;

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
    I.Y0 = r0 * ST - p.PH - R;  // window origin in input coordinates
    I.X0 = c0 * ST - p.PW - R;
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
  // Rows above and below the map fall out of the image's buffer range
  // (offsets relative to the image, negative ones wrapping past it); one
  // column check per slice rejects the columns beside it.
  auto issue_window = [&](const Item &I, bool valid) {
    const __amdgpu_buffer_rsrc_t rimg =
        make_rsrc(static_cast<const unsigned char *>(p.input) + I.img, img_bytes);
    const uint32_t base = (uint32_t)I.Y0 * row_bytes + (uint32_t)I.X0 * pix_bytes + I.chan;  // mod 2^32
    const uint32_t m_off = valid && (uint32_t)(I.X0 + (int)w_col) < (uint32_t)p.W ? base + w_lane : kOutOfRange;
#pragma unroll
    for (int u = 0; u < WS::NM; ++u)
      buffer_load_words<NWL>(rimg, m_off + (uint32_t)(u * WS::RPS) * row_bytes, win[u]);
#pragma unroll
    for (int rho = 0; rho < WS::NR; ++rho) {
      uint32_t y, x;
      const bool live = WS::rem(rho, quad, y, x);
      const uint32_t off = valid && live && (uint32_t)(I.X0 + (int)x) < (uint32_t)p.W
                               ? base + y * row_bytes + x * pix_bytes : kOutOfRange;
      buffer_load_words<NWL>(rimg, off, win[WS::NM + rho]);
    }
  };
  // (staged as fp32 whatever the I/O dtype)
  auto store_one = [&](uint32_t at, const uint32_t (&w)[NWL]) {
    float v[4];
    unpack<DT, NWL>(w, v);
    *reinterpret_cast<uint4 *>(lds + at) =
        make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
  };
  auto store_window = [&]() {
#pragma unroll
    for (int u = 0; u < WS::NM; ++u) store_one(w_lds + (uint32_t)(u * WS::RPS * ROW), win[u]);
#pragma unroll
    for (int rho = 0; rho < WS::NR; ++rho) {
      uint32_t y, x;
      if (WS::rem(rho, quad, y, x)) store_one((y * SPAN_W + x) * PIXB + sub * 16u, win[WS::NM + rho]);
    }
  };
  // Raw rows as loaded (decoded where used).  fp32: rw = x, y of k = 2 sub;
  // x, y of 2 sub + 1; x, y of 8; rl = logits of 2 sub, 2 sub + 1, 2 sub + 2
  // (lane 3: logit 8; with RC logits 2 sub, 2 sub + 1 and 0); rg =
  // grad_output of the lane's 4 channels.  16-bit: rw = (x, y) words of
  // 2 sub, 2 sub + 1, 8; rl = the three logits (low halves); rg = two words.
  constexpr int NRW = DT == DCN_F32 ? 2 * P : P;
  uint32_t rw[NRW], rl[P], rg[NWL];
  auto issue_rows = [&](const Item &I) {
    if constexpr (KS == 5) {  // one point at a time: the lane's P points, k = P sub + r (none past K)
#pragma unroll
      for (int r = 0; r < P; ++r) {
        const bool has = P * (int)sub + r < K;
        const uint32_t k = (uint32_t)(P * (int)sub + r);
        if constexpr (DT == DCN_F32) {
          const auto o = __builtin_amdgcn_raw_buffer_load_b64(
              roff, has ? (int)(I.pg * (uint32_t)(K * 8) + 8u * k) : (int)kOutOfRange, 0, 0);
          rw[2 * r] = o[0];
          rw[2 * r + 1] = o[1];
          rl[r] = __builtin_amdgcn_raw_buffer_load_b32(
              rmask, has ? (int)(I.pg * (uint32_t)(K * 4) + 4u * k) : (int)kOutOfRange, 0, 0);
        } else {
          rw[r] = __builtin_amdgcn_raw_buffer_load_b32(
              roff, has ? (int)(I.pg * (uint32_t)(K * 4) + 4u * k) : (int)kOutOfRange, 0, 0);
          rl[r] = __builtin_amdgcn_raw_buffer_load_b16(
              rmask, has ? (int)(I.pg * (uint32_t)(K * 2) + 2u * k) : (int)kOutOfRange, 0, 0);
        }
      }
      buffer_load_words<NWL>(rgy, I.pg * (uint32_t)(CG * EB) + sub * (uint32_t)LB, rg);
      return;
    }
    if constexpr (DT == DCN_F32) {
      const uint32_t orow = I.pg * (K * 8), mrow = I.pg * (K * 4);
      const auto o = __builtin_amdgcn_raw_buffer_load_b128(roff, (int)(orow + 16 * sub), 0, 0);
      if constexpr (RC) {
        const auto lg = __builtin_amdgcn_raw_buffer_load_b64(rmask, (int)(mrow + 8 * sub), 0, 0);
        rw[4] = rw[5] = rl[2] = 0u;
        rl[0] = lg[0];
        rl[1] = lg[1];
      } else {
        // logits 2 sub, 2 sub + 1, 2 sub + 2 in one load: lane 3's third is
        // logit 8, which lane 0 takes from it by DPP when the rows are decoded
        // (one row load fewer per lane than a separate load of logit 8)
        const auto lg = __builtin_amdgcn_raw_buffer_load_b96(rmask, (int)(mrow + 8 * sub), 0, 0);
        const auto o8 = __builtin_amdgcn_raw_buffer_load_b64(roff, (int)(orow + 64), 0, 0);
        rw[4] = o8[0];
        rw[5] = o8[1];
        rl[0] = lg[0];
        rl[1] = lg[1];
        rl[2] = lg[2];
      }
      rw[0] = o[0];
      rw[1] = o[1];
      rw[2] = o[2];
      rw[3] = o[3];
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

    // Own slots: offsets, modulation weights (softmax over the quad's K
    // logits for DCNv3, the raw mask for DCNv4) and grad_output.
    float2 offs[P];
    float m[P], gy[4];
    float lgs[P];
    // whether slot r of this lane holds a point (3x3: slot 2 is lane 0's k = 8)
    auto has_slot = [&](int r) -> bool { return KS == 3 ? (r < 2 || (!RC && sub == 0)) : (P * (int)sub + r < K); };
    // offset of slot r from the raw row words (5x5: decoded where used, so
    // the words stay the only copy)
    auto slot_offset = [&](int r) -> float2 {
      if constexpr (DT == DCN_F32)
        return make_float2(__uint_as_float(rw[2 * r]), __uint_as_float(rw[2 * r + 1]));
      else
        return make_float2(io::lo(rw[r]), io::hi(rw[r]));
    };
    if constexpr (KS == 3 && DT == DCN_F32 && !RC) rl[2] = (uint32_t)qbcast<3>((int)rl[2]);  // logit 8 from lane 3
#pragma unroll
    for (int r = 0; r < P; ++r) {
      if constexpr (KS == 3) offs[r] = slot_offset(r);
      lgs[r] = has_slot(r) ? io::lo(rl[r]) : (SOFTMAX ? -INFINITY : 0.f);
    }
    unpack<DT, NWL>(rg, gy);
    // grad_output in the scatter's pair order
    const float gys[4] = {podd ? gy[2] : gy[0], podd ? gy[3] : gy[1], podd ? gy[0] : gy[2], podd ? gy[1] : gy[3]};
    if constexpr (SOFTMAX) {
      float mx = lgs[0];
#pragma unroll
      for (int r = 1; r < P; ++r) mx = fmaxf(mx, lgs[r]);
      mx = quad_max(mx);
      float e[P], sum = 0.f;
#pragma unroll
      for (int r = 0; r < P; ++r) {
        e[r] = has_slot(r) ? __expf(lgs[r] - mx) : 0.f;
        sum += e[r];
      }
      const float inv = __builtin_amdgcn_rcpf(quad_sum(sum));
#pragma unroll
      for (int r = 0; r < P; ++r) m[r] = e[r] * inv;
    } else {
#pragma unroll
      for (int r = 0; r < P; ++r) m[r] = lgs[r];
    }

    // Fixed-point scale of the item's grad window.  A pixel-group adds at
    // most b = sum_k |m_k| * max_c |gy_c| to any window pixel-channel (the
    // four corner weights of a sample are non-negative and add up to 1), so
    // every partial sum there is at most B = the sum of b over the tile.
    // With S = 2^(30 - e), B <= 2^e, the scaled partial sums stay within
    // 2^30 and the LDS integer adds sum them exactly; each term is rounded to
    // the nearest multiple of 1/S, so an element that receives n terms is off
    // by at most n * 2^(e - 31) <= n * B * 2^-30.  That bound is set by the
    // whole tile, so the item takes fixed point only where it is small
    // against every contributor: B <= 2^12 * (the smallest nonzero b of the
    // tile), which keeps the error within n * 2^-18 of the bound b of each
    // pixel-group whose samples reach the element.  Tiles with a wider spread
    // (an outlier in grad_output or the mask) and a non-finite B (NaN or Inf
    // there) send the whole item to fp32 global atomics instead.
    {
      float gmax = 0.f, nanflag = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        gmax = fmaxf(gmax, fabsf(gy[c]));
        nanflag += 0.f * gy[c];  // fmaxf drops NaN: a NaN in gy must still reach the bound
      }
      float mabs = 0.f;
#pragma unroll
      for (int r = 0; r < P; ++r) mabs += fabsf(m[r]);
      const float msum = quad_sum(mabs);
      float bound = quad_max(gmax) * msum + quad_sum(nanflag);
      bound = (cur.live && sub == 0) ? bound : 0.f;
      float bmin = bound > 0.f ? bound : INFINITY;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        bound += __shfl_xor(bound, d, 64);
        bmin = fminf(bmin, __shfl_xor(bmin, d, 64));
      }
      if ((threadIdx.x & 63) == 0) {
        wave_sums[threadIdx.x >> 6] = bound;
        wave_mins[threadIdx.x >> 6] = bmin;
      }
    }
    __syncthreads();  // the window is in LDS, the wave bounds are ready

    float B = 0.f, bmin = INFINITY;
#pragma unroll
    for (int wv = 0; wv < G::kWaves; ++wv) {
      B += wave_sums[wv];
      bmin = fminf(bmin, wave_mins[wv]);
    }
    // false for Inf and NaN, and for a spread above 2^12 (block-uniform)
    const bool fixed = B <= 3.0e38f && B <= kFixedSpread * bmin;
    int ex = 0;
    frexpf(B, &ex);
    ex = ex < -96 ? -96 : ex;
    // (an item off fixed point keeps its weights unscaled: S = 1)
    const float S = fixed ? ldexpf(1.f, 30 - ex) : 1.f, invS = fixed ? ldexpf(1.f, ex - 30) : 1.f;

    const uint32_t next = item + walk.stride;
    const bool more = next < end;  // block-uniform
    const Item nx = decode(more ? next : item);
    issue_window(nx, more);
    if constexpr (KS == 3) issue_rows(nx);  // 5x5: after the rounds, which read the current rows

    // One round: every lane's point of slot r (its offset o2 and weight mk,
    // its window position (bx, by) before the offset), processed by the
    // whole quad; `owners` of the quad's lanes hold a point this round.
    // Returns the owner's (gm, d/dx, d/dy).
    auto round = [&](int r, float2 o2, float mk, int bx, int by, int owners) -> float3 {
      // Wave priority falls round by round: the waves furthest behind issue
      // first, so the block reaches its flush barrier with less spread.
      if (r == 0) __builtin_amdgcn_s_setprio(3);
      if (r == (KS == 3 ? 1 : P / 3)) __builtin_amdgcn_s_setprio(2);
      if (r == (KS == 3 ? 2 : 2 * P / 3)) __builtin_amdgcn_s_setprio(1);
      const float dx = s * o2.x, dy = s * o2.y;
      const bool nan_loc = (dx != dx) | (dy != dy);
      const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
      const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
      const float fx = floorf(cx), fy = floorf(cy);
      const float lx = cx - fx, ly = cy - fy;
      const float hx = 1.f - lx, hy = 1.f - ly;
      const int tx = bx + (int)fx;  // window coordinates
      const int ty = by + (int)fy;
      const bool inside = cur.live && !nan_loc && (uint32_t)ty <= (uint32_t)LIM_Y && (uint32_t)tx <= (uint32_t)LIM_X;
      const uint32_t A = inside ? mad24((uint32_t)ty, (uint32_t)ROW, mul24((uint32_t)tx, PIXB)) : ZERO;
      const float wy1 = ly * mk, wy0 = mk - wy1;
      const float W1 = wy0 * lx, W0 = wy0 - W1;
      const float W3 = wy1 * lx, W2 = wy1 - W3;
      // scaled to the fixed-point grid for the LDS scatter (the global path
      // scales them back: powers of two, so exactly)
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
      // 3x3: the quad's corner sums of this lane's own point, turned into
      // its results once per round; 5x5 (whose tiles leave fewer registers):
      // the owner's results directly.
      float Gown[4] = {0.f, 0.f, 0.f, 0.f};
      float3 mine = make_float3(0.f, 0.f, 0.f);

      // gm, d/dx and d/dy of the own point from the quad's corner sums G (00,
      // 01, 10, 11): one-sided derivatives of the bilinear form, linear in G.
      auto own_results = [&](const float (&G)[4]) -> float3 {
        const float T = hx * G[0] + lx * G[1], Bt = hx * G[2] + lx * G[3];
        return nan_loc ? make_float3(qnan, qnan, qnan)
                       : make_float3(hy * T + ly * Bt, hy * (G[1] - G[0]) + ly * (G[3] - G[2]), Bt - T);
      };

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
        // owner keeps them (3x3: selects, no branch) or its results.
        quad_sum4(P);
        if constexpr (KS == 3) {
          const bool owner = sub == (uint32_t)O;
#pragma unroll
          for (int q = 0; q < 4; ++q) Gown[q] = owner ? P[q] : Gown[q];
        } else if (sub == (uint32_t)O) {
          mine = own_results(P);
        }
        // Scatter m_k * w_corner * gy_c of this lane's 4 channels (no
        // branch: samples the window does not hold add into the sink).
        if (fixed) {  // block-uniform
          const uint32_t d = add_bcast<O>(AS, gwin_chunk);  // the lane's first pair
          const uint32_t d2 = ALT ? (d ^ 8u) : d + 8u;              // and its second
          auto corner = [&](float w, uint32_t off) {
            float t[4];
            mul4_bcast<O>(t, w, gys);
            lds_add_pair(d + off, cvt_rpi(t[0]), cvt_rpi(t[1]));
            lds_add_pair(d2 + off, cvt_rpi(t[2]), cvt_rpi(t[3]));
          };
          corner(W0s, 0u);
          corner(W1s, PIXB);
          corner(W2s, ROW);
          corner(W3s, ROW + PIXB);
        }
        if (gs_any) {
          if (qbcast<O>((int)gscat)) {
            uint32_t ga[4];
            corners(ga);
            const float wc[4] = {qbcast<O>(W0s) * invS, qbcast<O>(W1s) * invS, qbcast<O>(W2s) * invS,
                                 qbcast<O>(W3s) * invS};
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
      if (owners > 1) point(I1{});
      if (owners > 2) point(I2{});
      if (owners > 3) point(I3{});
      // 3x3: once per round in every lane (a lane without a point this round
      // returns values nobody stores)
      if constexpr (KS == 3) mine = own_results(Gown);
      return mine;
    };

    // (gm, d/dx, d/dy) of the own slots
    float3 res[P];
    if constexpr (KS == 3) {
      // Slot inputs shifted in round by round; after the three rounds (two
      // with RC, then one empty shift) res2 holds slot 0, res1 slot 1, res0
      // slot 2.  The last round holds only k = 8 (owner lane 0).
      float3 res0 = make_float3(0.f, 0.f, 0.f), res1 = res0, res2 = res0;
      float2 o2 = offs[0], o2n = offs[1], o2nn = offs[2];
      float mk = m[0], mkn = m[1], mknn = m[2];
#pragma unroll 1
      for (int r = 0; r < ROUNDS; ++r) {
        const float3 mine = round(r, o2, mk, (int)((bxp >> (10 * r)) & 1023u), (int)((byp >> (10 * r)) & 1023u),
                                  r < 2 ? 4 : 1);
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
      res[0] = res2;
      res[1] = res1;
      res[2] = res0;
    } else {
      // The offset gradients of each slot are stored as its round ends (they
      // need no other slot); gm waits for the softmax Jacobian.
#pragma unroll
      for (int r = 0; r < P; ++r) {
        const int k = P * (int)sub + r;
        const int q = RC ? k + (k >= KS * KS / 2) : k;  // grid index
        const int owners = (K - 1 - r) / P + 1 < 4 ? (K - 1 - r) / P + 1 : 4;
        const float3 mine = round(r, slot_offset(r), m[r], ox + R + q % KS, oy + R + q / KS, owners);
        res[r] = make_float3(mine.x, 0.f, 0.f);
        const bool put = cur.live && has_slot(r);
        const float gx_ = s * m[r] * mine.y, gy_ = s * m[r] * mine.z;
        if constexpr (DT == DCN_F32) {
          typedef float f2 __attribute__((ext_vector_type(2)));
          __builtin_amdgcn_raw_buffer_store_b64(
              __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))), f2{gx_, gy_}), rgoff,
              put ? (int)(cur.pg * (uint32_t)(K * 8) + 8u * (uint32_t)k) : (int)kOutOfRange, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(
              io::pack(gx_, gy_), rgoff, put ? (int)(cur.pg * (uint32_t)(K * 4) + 4u * (uint32_t)k) : (int)kOutOfRange,
              0, 0);
        }
      }
      issue_rows(nx);
    }

    // Offset and mask gradients of the own slots (a NaN sampling location
    // makes its point's offset gradient and gm NaN).
    if (cur.live) {
      float gm[P];
#pragma unroll
      for (int r = 0; r < P; ++r) gm[r] = res[r].x;
      if constexpr (SOFTMAX) {
        float dot = 0.f;
#pragma unroll
        for (int r = 0; r < P; ++r)
          if (has_slot(r)) dot += m[r] * gm[r];
        dot = quad_sum(dot);
#pragma unroll
        for (int r = 0; r < P; ++r) gm[r] = m[r] * (gm[r] - dot);
      }
      // offset gradients (x, y) of the slots
      float go[P][2];
#pragma unroll
      for (int r = 0; r < P; ++r) {
        go[r][0] = s * m[r] * res[r].y;
        go[r][1] = s * m[r] * res[r].z;
      }
      if constexpr (KS == 5) {  // gm, one point at a time (k = P sub + r), none past K
#pragma unroll
        for (int r = 0; r < P; ++r) {
          const bool has = has_slot(r);
          const uint32_t k = (uint32_t)(P * (int)sub + r);
          if constexpr (DT == DCN_F32)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gm[r]), rgm,
                                                  has ? (int)(cur.pg * (uint32_t)(K * 4) + 4u * k) : (int)kOutOfRange, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(io::pack(gm[r], 0.f) & 0xffffu), rgm,
                                                  has ? (int)(cur.pg * (uint32_t)(K * 2) + 2u * k) : (int)kOutOfRange, 0, 0);
        }
      } else if constexpr (DT == DCN_F32) {
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
    // 64-byte request), and clear it for the next item.  Zero sums are
    // skipped; rows outside the map fall out of the image's buffer range,
    // columns beside it are rejected per slice.
    {
      const uint32_t ch = threadIdx.x & 15u, fg = threadIdx.x >> 4;  // channel, lane group
      const __amdgpu_buffer_rsrc_t rgimg =
          make_rsrc(static_cast<unsigned char *>(bp.grad_in) + (size_t)cur.img * GX, img_bytes * GX);
      // grad_input offset (in input bytes, relative to the image, mod 2^32)
      // of window pixel (0, 0), channel ch of the group
      const uint32_t base = (uint32_t)cur.Y0 * row_bytes + (uint32_t)cur.X0 * pix_bytes +
                            cur.g * (uint32_t)(CG * EB) + ch * (uint32_t)EB;
      const uint32_t pair = GWIN + (ch >> 1) * 8u;
      typedef __attribute__((address_space(3))) uint64_t L;
      auto flush_one = [&](uint32_t lds_at, uint32_t dst, bool ok) {
        L *slot = (L *)(size_t)(lbase + lds_at);
        const int2 pr = pair_sums(*slot);
        *slot = 0;  // both lanes of the pair, after both have read it (the read is the earlier instruction)
        const int q = (ch & 1u) ? pr.y : pr.x;
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32((float)q * invS, rgimg,
                                                        (int)((ok && q != 0) ? dst * GX : kOutOfRange), 0, 0);
      };
      const uint32_t f_col = fg % (uint32_t)FS::CW, f_row = fg / (uint32_t)FS::CW;
      const bool f_ok = (uint32_t)(cur.X0 + (int)f_col) < (uint32_t)p.W;
      const uint32_t f_dst = base + f_row * row_bytes + f_col * pix_bytes;
      const uint32_t f_lds = pair + (f_row * SPAN_W + f_col) * PIXB;
#pragma unroll 4
      for (int u = 0; u < FS::NM; ++u)
        flush_one(f_lds + (uint32_t)(u * FS::RPS * ROW), f_dst + (uint32_t)(u * FS::RPS) * row_bytes, f_ok);
#pragma unroll
      for (int rho = 0; rho < FS::NR; ++rho) {
        uint32_t y, x;
        if (FS::rem(rho, fg, y, x))
          flush_one(pair + (y * SPAN_W + x) * PIXB, base + y * row_bytes + x * pix_bytes,
                    (uint32_t)(cur.X0 + (int)x) < (uint32_t)p.W);
      }
    }

    item = next;
    cur = nx;
  }
}

namespace {

template <int DT, bool SM, bool RC, int DIL, int TW, int TH, int ST, int KS>
hipError_t launch_bwd_quad(const BwdParams &p, const TileGeom &tg, hipStream_t s) {
  using G = BqGeom<TW, TH, ST, KS>;
  auto kern = dcn_bwd_quad_kernel<DT, SM, RC, DIL, TW, TH, ST, KS>;
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

template <bool RC, int DIL, int TW, int TH, int ST = 1, int KS = 3>
hipError_t launch_dt(int dtype, int softmax, const BwdParams &b, const TileGeom &tg, hipStream_t s) {
  switch (dtype) {
    case DCN_F32:
      return softmax ? launch_bwd_quad<DCN_F32, true, RC, DIL, TW, TH, ST, KS>(b, tg, s)
                     : launch_bwd_quad<DCN_F32, false, RC, DIL, TW, TH, ST, KS>(b, tg, s);
    case DCN_F16:
      return softmax ? launch_bwd_quad<DCN_F16, true, RC, DIL, TW, TH, ST, KS>(b, tg, s)
                     : launch_bwd_quad<DCN_F16, false, RC, DIL, TW, TH, ST, KS>(b, tg, s);
    case DCN_BF16:
      return softmax ? launch_bwd_quad<DCN_BF16, true, RC, DIL, TW, TH, ST, KS>(b, tg, s)
                     : launch_bwd_quad<DCN_BF16, false, RC, DIL, TW, TH, ST, KS>(b, tg, s);
    default: return hipErrorInvalidValue;
  }
}

// The same for shapes only taken with 16-bit I/O.
template <bool RC, int DIL, int TW, int TH, int ST, int KS>
hipError_t launch_16bit(int dtype, int softmax, const BwdParams &b, const TileGeom &tg, hipStream_t s) {
  switch (dtype) {
    case DCN_F16:
      return softmax ? launch_bwd_quad<DCN_F16, true, RC, DIL, TW, TH, ST, KS>(b, tg, s)
                     : launch_bwd_quad<DCN_F16, false, RC, DIL, TW, TH, ST, KS>(b, tg, s);
    case DCN_BF16:
      return softmax ? launch_bwd_quad<DCN_BF16, true, RC, DIL, TW, TH, ST, KS>(b, tg, s)
                     : launch_bwd_quad<DCN_BF16, false, RC, DIL, TW, TH, ST, KS>(b, tg, s);
    default: return hipErrorInvalidValue;
  }
}

// Share of the tiles' pixels that are output pixels.
double quad_tile_use(const FwdParams &p, int tw, int th) {
  const double tiled = (double)((p.Ho + th - 1) / th) * th * (double)((p.Wo + tw - 1) / tw) * tw;
  return (double)p.Ho * p.Wo / tiled;
}

}  // namespace

// 3x3 points (all nine, or eight without the centre) at stride 1 or 2 and
// dilation 1 or 2 (each the same on both axes), and 5x5 points (25 or 24)
// at stride and dilation 1, on tiles of 8 to 16 rows; hipErrorNotSupported
// otherwise.
hipError_t launch_backward_quad(int dtype, int softmax, const BwdParams &b, hipStream_t s) {
  const FwdParams &p = b.f;
  const bool k5 = p.KH == 5 && p.KW == 5 && p.SH == 1 && p.SW == 1 && p.DH == 1 && p.DW == 1;
  if (!k5 && (p.KH != 3 || p.KW != 3 || p.SH != p.SW || (p.SH != 1 && p.SH != 2) || p.DH != p.DW ||
              (p.DH != 1 && p.DH != 2)))
    return hipErrorNotSupported;
  const bool s2 = p.SH == 2;
  // 24x8 or 12x12 tiles (stride and dilation 1) where they leave clearly
  // fewer quads idle than 16x16 ones (24x8 on a tie between the two)
  const double u16 = quad_tile_use(p, 16, 16), u24 = quad_tile_use(p, 24, 8), u12 = quad_tile_use(p, 12, 12);
  const bool wide = !k5 && !s2 && p.DH == 1 && u24 > u16 + 0.1 && u24 >= u12;
  const bool small = !k5 && !s2 && p.DH == 1 && !wide && u12 > u16 + 0.1;
  // 5x5 points: 16x8 tiles in fp32 (16x16 ones spill at 1024 threads) and
  // where they leave clearly fewer quads idle, 16x16 tiles otherwise
  const bool k5_tall = k5 && dtype != DCN_F32 && quad_tile_use(p, 16, 8) <= u16 + 0.1;
  const int tw = wide ? 24 : (small ? 12 : 16),
            th = k5 ? (k5_tall ? 16 : 8) : (s2 || wide ? 8 : (small ? 12 : 16));
  TileGeom tg{};
  tg.span_w = s2 ? BqGeom<16, 8, 2>::kSpanW
                 : (k5 ? (k5_tall ? BqGeom<16, 16, 1, 5>::kSpanW : BqGeom<16, 8, 1, 5>::kSpanW)
                       : tw + 2 * kBqHalo + 3);
  tg.span_h = s2 ? BqGeom<16, 8, 2>::kSpanH
                 : (k5 ? (k5_tall ? BqGeom<16, 16, 1, 5>::kSpanH : BqGeom<16, 8, 1, 5>::kSpanH)
                       : th + 2 * kBqHalo + 3);
  // Window rows outside the map are rejected by the buffer range of their
  // image (input, and grad_input at GX bytes per input byte), which needs
  // every window row's offset relative to the image to fit int32.
  const int64_t row_bytes = (int64_t)p.W * p.C * (dtype == DCN_F32 ? 4 : 2);
  const int64_t gx = dtype == DCN_F32 ? 1 : 2;
  if (((int64_t)p.H + p.PH + tg.span_h + 1) * row_bytes * gx >= (int64_t(1) << 31)) return hipErrorNotSupported;
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
  if (k5_tall)
    return p.RC ? launch_16bit<true, 1, 16, 16, 1, 5>(dtype, softmax, b, tg, s)
                : launch_16bit<false, 1, 16, 16, 1, 5>(dtype, softmax, b, tg, s);
  if (k5)
    return p.RC ? launch_dt<true, 1, 16, 8, 1, 5>(dtype, softmax, b, tg, s)
                : launch_dt<false, 1, 16, 8, 1, 5>(dtype, softmax, b, tg, s);
  if (s2 && p.DH == 2)
    return p.RC ? launch_dt<true, 2, 16, 8, 2>(dtype, softmax, b, tg, s) : launch_dt<false, 2, 16, 8, 2>(dtype, softmax, b, tg, s);
  if (s2)
    return p.RC ? launch_dt<true, 1, 16, 8, 2>(dtype, softmax, b, tg, s) : launch_dt<false, 1, 16, 8, 2>(dtype, softmax, b, tg, s);
  if (p.DH == 2)
    return p.RC ? launch_dt<true, 2, 16, 16>(dtype, softmax, b, tg, s) : launch_dt<false, 2, 16, 16>(dtype, softmax, b, tg, s);
  if (wide)
    return p.RC ? launch_dt<true, 1, 24, 8>(dtype, softmax, b, tg, s) : launch_dt<false, 1, 24, 8>(dtype, softmax, b, tg, s);
  if (small)
    return p.RC ? launch_dt<true, 1, 12, 12>(dtype, softmax, b, tg, s) : launch_dt<false, 1, 12, 12>(dtype, softmax, b, tg, s);
  return p.RC ? launch_dt<true, 1, 16, 16>(dtype, softmax, b, tg, s) : launch_dt<false, 1, 16, 16>(dtype, softmax, b, tg, s);
}

}  // namespace dcn
