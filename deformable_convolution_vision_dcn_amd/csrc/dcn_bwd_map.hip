// dcn_bwd_map.hip -- whole-map gfx950 backward kernel of the DCN core for
// small feature maps (fp32 arithmetic for fp32 and 16-bit I/O): 3x3 kernel
// points at dilation 1 and stride 1 (the InternImage configuration;
// wmrh.cn/news/61976, section 二 steps 2-4 and section 三) or 2 (the DCNv4
// signature carries the stride), all nine points or the eight left by
// DCNv4's remove_center (pnsm.cn/news/2029644.html section 3.3).
//
// The derivatives are those of the tiled kernels: every in-map corner of a
// sample receives m_k * w_corner * gy_c; the offset gradient is
// s * m_k * sum_c gy_c * dB_k[c]/d(px, py) (one-sided from the right at
// integer coordinates); the mask gradient is gm_k = sum_c gy_c * B_k[c],
// through the softmax Jacobian for DCNv3.
//
// Layout of the work: persistent blocks, each walking (image, group) items.
// A block owns the item's whole grad_input slice: it stages the group's
// input map with a one-pixel zero border in LDS, runs the item's output
// pixels in NP passes of TW x TH (a lane quad per pixel-group, as in the
// tiled kernels) and sums every scatter into a fixed-point grad window of the
// same shape.  No other block touches that slice, so the window is written
// to grad_input once, rounded to the I/O dtype, with plain stores: no
// clearing of grad_input before the call, no global atomics, no fp32
// accumulator for 16-bit I/O.  A sample whose corners are all off the map
// contributes nothing and adds into a sink.  An item whose terms are too
// spread for fixed point (or not finite) clears its slice of the fp32
// accumulator `acc`, adds its terms there with fp32 atomics and, for 16-bit
// I/O, rounds the slice into grad_input at the end.
#include <algorithm>
#include <type_traits>

#include "bwd_fixed.hpp"
#include "dcn_device.hpp"
#include "index_math.hpp"
#include "quad_ops.hpp"

namespace dcn {

constexpr int kBmPixB = 64;  // 16 fp32 channels of a window pixel

// TW x TH output pixels per pass (a quad per pixel), NP passes, at stride
// ST; the window holds an input map of up to ST*TW x ST*NP*TH pixels and its
// border.
template <int TW, int TH, int NP, int ST>
struct BmGeom {
  static_assert(ST == 1 || ST == 2, "stride 1 or 2");
  static constexpr int kThreads = 4 * TW * TH;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kSpanW = ST * TW + 2, kSpanH = ST * NP * TH + 2;
  static constexpr int kRow = kSpanW * kBmPixB;
  static constexpr int kWin = kSpanW * kSpanH * kBmPixB;
  static constexpr int kZero = kRow + 2 * kBmPixB;  // zero block after the input window
  static constexpr int kSink = kRow + 2 * kBmPixB;  // scatter sink after the grad window
  static constexpr size_t kLds = (size_t)kWin + kZero + kWin + kSink + 8 * kWaves;
  static_assert(kThreads % 64 == 0 && kThreads <= 1024, "block size");
};

// RC: the centre point is removed (8 points, k -> grid index k + (k >= 4)):
// each lane owns exactly two points and a pass takes two rounds instead of
// three.
template <int DT, bool SOFTMAX, bool RC, int TW, int TH, int NP, int ST>
__global__ void __launch_bounds__(4 * TW * TH, 1) dcn_bwd_map_kernel(BwdParams bp, TileGeom tg) {
  using G = BmGeom<TW, TH, NP, ST>;
  const FwdParams &p = bp.f;
  using io = Io<DT>;
  constexpr int EB = io::kBytes;         // bytes per element in memory
  constexpr int LB = 4 * EB;             // a lane's 4 channels in memory
  constexpr int NWL = LB / 4;            // words of them: 4 (fp32) or 2 (16-bit)
  constexpr uint32_t GX = 4 / EB;        // input byte offset -> fp32 accumulator byte offset
  constexpr int SPAN_W = G::kSpanW, SPAN_H = G::kSpanH;
  constexpr int PIXB = kBmPixB, ROW = G::kRow, LIM_X = SPAN_W - 2, LIM_Y = SPAN_H - 2;
  constexpr int CG = kGroupChannels, K = 9 - (RC ? 1 : 0);
  constexpr int P = 3;                   // slots per lane: k = 2 sub, 2 sub + 1 and (lane 0) 8
  constexpr int ROUNDS = RC ? 2 : 3;
  constexpr int WPIX = G::kThreads / 4;  // window pixels per staging slice
  using WS = Slices<SPAN_W, SPAN_H, WPIX>;
  constexpr int SLOTS = WS::N;
  constexpr uint32_t ZERO = G::kWin;               // zero block (reads of samples off the map)
  constexpr uint32_t GWIN = G::kWin + G::kZero;    // fixed-point grad window
  constexpr uint32_t SINK = GWIN + G::kWin;        // scatter target of samples off the map
  static_assert(CG == 16, "a quad covers 16 channels");

  extern __shared__ __align__(16) unsigned char lds[];
  typedef __attribute__((address_space(3))) unsigned char lds_byte;
  const uint32_t lbase = (uint32_t)(size_t)(lds_byte *)lds;
  float *wave_sums = reinterpret_cast<float *>(lds + SINK + G::kSink);
  float *wave_mins = wave_sums + G::kWaves;

  const uint32_t quad = threadIdx.x >> 2, sub = threadIdx.x & 3;
  const int oy = (int)quad / TW, ox = (int)quad % TW;  // output pixel within a pass
  const uint32_t pix_bytes = (uint32_t)p.C * EB;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const uint32_t img_bytes = (uint32_t)p.H * row_bytes;
  const __amdgpu_buffer_rsrc_t roff = make_rsrc(p.offset, p.off_bytes);
  const __amdgpu_buffer_rsrc_t rmask = make_rsrc(p.mask, p.mask_bytes);
  const __amdgpu_buffer_rsrc_t rgy = make_rsrc(bp.grad_out, p.pg_total * (uint32_t)(CG * EB));
  const __amdgpu_buffer_rsrc_t rgoff = make_rsrc(bp.grad_offset, p.off_bytes);
  const __amdgpu_buffer_rsrc_t rgm = make_rsrc(bp.grad_mask, p.mask_bytes);
  const float s = p.scale;
  const float qnan = __builtin_nanf("");

  // This quad's input-window slices (main: row w_row + u RPS, column w_col).
  const uint32_t w_col = quad % (uint32_t)WS::CW, w_row = quad / (uint32_t)WS::CW;
  const uint32_t w_lane = w_row * row_bytes + w_col * pix_bytes;
  const uint32_t w_lds = (w_row * SPAN_W + w_col) * PIXB + sub * 16u;

  // Window position of each own slot's kernel point before its offset in
  // pass 0 (window pixel (y, x) is input pixel (y - 1, x - 1)); a pass moves
  // it down by ST * TH rows.
  int bx[P], by[P];
#pragma unroll
  for (int r = 0; r < P; ++r) {
    const int k = r < 2 ? 2 * (int)sub + r : 8;
    const int q = RC ? (r < 2 ? k + (k >= 4) : 4) : k;
    bx[r] = ox * ST - p.PW + q % 3 + 1;
    by[r] = oy * ST - p.PH + q / 3 + 1;
  }
  const uint32_t win_chunk = lbase + sub * 16u;  // this lane's 4 channels of a window pixel
  // The scatter's first 64-bit add of a corner takes the lane's first channel
  // pair in even quads and its second pair in odd ones, so the four quads of
  // a 16-lane group spread over twice as many LDS banks (the layout is the
  // same: pair 0 at +0, pair 1 at +8 of the lane's 16 bytes).
  const uint32_t podd = quad & 1u;
  const uint32_t gwin_chunk = lbase + GWIN + sub * 16u + 8u * podd;

  // The grad window starts at zero; every item's flush clears it again.  The
  // zero block after the input window is written once.
  for (uint32_t z = threadIdx.x * 16u; z < (uint32_t)G::kWin; z += G::kThreads * 16u)
    *reinterpret_cast<uint4 *>(lds + GWIN + z) = make_uint4(0, 0, 0, 0);
  for (uint32_t z = threadIdx.x * 16u; z < (uint32_t)G::kZero; z += G::kThreads * 16u)
    *reinterpret_cast<uint4 *>(lds + ZERO + z) = make_uint4(0, 0, 0, 0);

  struct Item {
    uint32_t g, n, img, chan;
  };
  auto decode = [&](uint32_t it) {
    Item I;
    I.n = fast_div(it, tg.div_g);
    I.g = it - I.n * (uint32_t)p.G;
    I.img = I.n * img_bytes;
    I.chan = I.g * (uint32_t)(CG * EB) + sub * (uint32_t)LB;
    return I;
  };
  // pixel-group of this quad in pass pp, and whether it is an output pixel
  auto pass_pg = [&](const Item &I, int pp, bool &live) -> uint32_t {
    const int ho = pp * TH + oy;
    live = ho < p.Ho && ox < p.Wo;
    return live ? ((I.n * (uint32_t)p.Ho + (uint32_t)ho) * (uint32_t)p.Wo + (uint32_t)ox) * (uint32_t)p.G + I.g
                : 0u;
  };

  // Next item's input window (4 lanes of 16 bytes per pixel), requested into
  // registers while the current item computes.  Rows above and below the map
  // fall out of the image's buffer range (offsets relative to the image,
  // negative ones wrapping past it); one column check per slice rejects the
  // columns beside it.
  uint32_t win[SLOTS][NWL];
  auto issue_window = [&](const Item &I, bool valid) {
    const __amdgpu_buffer_rsrc_t rimg = make_rsrc(static_cast<const unsigned char *>(p.input) + I.img, img_bytes);
    const uint32_t base = I.chan - row_bytes - pix_bytes;  // window (0, 0) = input (-1, -1), mod 2^32
    const uint32_t m_off = valid && (uint32_t)((int)w_col - 1) < (uint32_t)p.W ? base + w_lane : kOutOfRange;
#pragma unroll
    for (int u = 0; u < WS::NM; ++u)
      buffer_load_words<NWL>(rimg, m_off + (uint32_t)(u * WS::RPS) * row_bytes, win[u]);
#pragma unroll
    for (int rho = 0; rho < WS::NR; ++rho) {
      uint32_t y, x;
      const bool live = WS::rem(rho, quad, y, x);
      const uint32_t off = valid && live && (uint32_t)((int)x - 1) < (uint32_t)p.W
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

  // Raw rows of each pass as loaded (decoded where used).  fp32: rw = x, y of
  // k = 2 sub; x, y of 2 sub + 1; x, y of 8; rl = logits of 2 sub, 2 sub + 1,
  // 8; rg = grad_output of the lane's 4 channels.  16-bit: rw = (x, y) words
  // of 2 sub, 2 sub + 1, 8; rl = the three logits (low halves); rg = two
  // words.  Slot i holds the rows of the i-th pass ahead: the pass loop
  // reads slot 0, then shifts the slots down and requests the next item's
  // rows of the same pass into the last one.  Pixels that are not output
  // pixels load nothing (out of range reads zero).
  constexpr int NRW = DT == DCN_F32 ? 2 * P : P;
  uint32_t rw[NP][NRW], rl[NP][P], rg[NP][NWL];
  auto issue_rows = [&](const Item &I, int pp, bool valid, auto slot_tag) {
    constexpr int SL = decltype(slot_tag)::value;
    bool live;
    const uint32_t pg = pass_pg(I, pp, live);
    live = live && valid;
    if constexpr (DT == DCN_F32) {
      const uint32_t orow = pg * (K * 8), mrow = pg * (K * 4);
      const auto o = __builtin_amdgcn_raw_buffer_load_b128(roff, live ? (int)(orow + 16 * sub) : (int)kOutOfRange, 0, 0);
      const auto lg = __builtin_amdgcn_raw_buffer_load_b64(rmask, live ? (int)(mrow + 8 * sub) : (int)kOutOfRange, 0, 0);
      if constexpr (RC) {
        rw[SL][4] = rw[SL][5] = rl[SL][2] = 0u;
      } else {
        const auto o8 = __builtin_amdgcn_raw_buffer_load_b64(roff, live ? (int)(orow + 64) : (int)kOutOfRange, 0, 0);
        rl[SL][2] = __builtin_amdgcn_raw_buffer_load_b32(rmask, live ? (int)(mrow + 32) : (int)kOutOfRange, 0, 0);
        rw[SL][4] = o8[0];
        rw[SL][5] = o8[1];
      }
      rw[SL][0] = o[0];
      rw[SL][1] = o[1];
      rw[SL][2] = o[2];
      rw[SL][3] = o[3];
      rl[SL][0] = lg[0];
      rl[SL][1] = lg[1];
    } else {
      const uint32_t orow = pg * (K * 4), mrow = pg * (K * 2);
      const auto o = __builtin_amdgcn_raw_buffer_load_b64(roff, live ? (int)(orow + 8 * sub) : (int)kOutOfRange, 0, 0);
      rw[SL][0] = o[0];
      rw[SL][1] = o[1];
      if constexpr (RC) {  // 16-byte mask rows: the lane's two logits in one word
        const uint32_t lw = __builtin_amdgcn_raw_buffer_load_b32(rmask, live ? (int)(mrow + 4 * sub) : (int)kOutOfRange, 0, 0);
        rl[SL][0] = lw & 0xffffu;
        rl[SL][1] = lw >> 16;
        rw[SL][2] = rl[SL][2] = 0u;
      } else {
        rw[SL][2] = __builtin_amdgcn_raw_buffer_load_b32(roff, live ? (int)(orow + 32) : (int)kOutOfRange, 0, 0);
        rl[SL][0] = __builtin_amdgcn_raw_buffer_load_b16(rmask, live ? (int)(mrow + 4 * sub) : (int)kOutOfRange, 0, 0);
        rl[SL][1] = __builtin_amdgcn_raw_buffer_load_b16(rmask, live ? (int)(mrow + 4 * sub + 2) : (int)kOutOfRange, 0, 0);
        rl[SL][2] = __builtin_amdgcn_raw_buffer_load_b16(rmask, live ? (int)(mrow + 16) : (int)kOutOfRange, 0, 0);
      }
    }
    buffer_load_words<NWL>(rgy, live ? pg * (uint32_t)(CG * EB) + sub * (uint32_t)LB : kOutOfRange, rg[SL]);
  };

  // whether slot r of this lane holds a point (slot 2 is lane 0's k = 8)
  auto has_slot = [&](int r) -> bool { return r < 2 || (!RC && sub == 0); };
  // modulation weights of the own slots of pass pp (softmax over the quad's
  // K logits for DCNv3, the raw mask for DCNv4)
  auto weights = [&](auto slot_tag, float (&m)[P]) {
    constexpr int SL = decltype(slot_tag)::value;
    float lgs[P];
#pragma unroll
    for (int r = 0; r < P; ++r) lgs[r] = has_slot(r) ? io::lo(rl[SL][r]) : (SOFTMAX ? -INFINITY : 0.f);
    if constexpr (SOFTMAX) {
      float mx = fmaxf(fmaxf(lgs[0], lgs[1]), lgs[2]);
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
  };

  const XcdWalk walk = xcd_walk(blockIdx.x, gridDim.x, tg.items);
  const uint32_t end = walk.end;
  uint32_t item = walk.first;
  Item cur = decode(item < end ? item : 0);
  if (item < end) {
    issue_window(cur, true);
    issue_rows(cur, 0, true, std::integral_constant<int, 0>{});
    if constexpr (NP > 1) issue_rows(cur, 1, true, std::integral_constant<int, (NP > 1 ? 1 : 0)>{});
    if constexpr (NP > 2) issue_rows(cur, 2, true, std::integral_constant<int, (NP > 2 ? 2 : 0)>{});
  }

  while (item < end) {
    __syncthreads();  // the previous item's reads, scatters and flush are done
    store_window();

    // Fixed-point scale of the item's grad window.  A pixel-group adds at
    // most b = sum_k |m_k| * max_c |gy_c| to any window pixel-channel (the
    // four corner weights of a sample are non-negative and add up to 1), so
    // every partial sum there is at most B = the sum of b over the map.
    // With S = 2^(30 - e), B <= 2^e, the scaled partial sums stay within
    // 2^30 and the LDS integer adds sum them exactly; each term is rounded to
    // the nearest multiple of 1/S, so an element that receives n terms is off
    // by at most n * 2^(e - 31) <= n * B * 2^-30.  The item takes fixed point
    // only where that is small against every contributor: B <= 2^12 * (the
    // smallest nonzero b of the map), which keeps the error within n * 2^-18
    // of the bound b of each pixel-group whose samples reach the element.
    // Items with a wider spread (an outlier in grad_output or the mask) and a
    // non-finite B (NaN or Inf there) take fp32 atomics instead.
    {
      float bound = 0.f, bmin = INFINITY;
      auto pass_bound = [&](auto slot_tag) {
        constexpr int pp = decltype(slot_tag)::value;
        bool live;
        (void)pass_pg(cur, pp, live);
        float gy[4];
        unpack<DT, NWL>(rg[pp], gy);
        float gmax = 0.f, nanflag = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          gmax = fmaxf(gmax, fabsf(gy[c]));
          nanflag += 0.f * gy[c];  // fmaxf drops NaN: a NaN in gy must still reach the bound
        }
        float m[P];
        weights(slot_tag, m);
        float mabs = 0.f;
#pragma unroll
        for (int r = 0; r < P; ++r) mabs += fabsf(m[r]);
        float b = quad_max(gmax) * quad_sum(mabs) + quad_sum(nanflag);
        b = (live && sub == 0) ? b : 0.f;
        bound += b;
        bmin = fminf(bmin, b > 0.f ? b : INFINITY);
      };
      pass_bound(std::integral_constant<int, 0>{});
      if constexpr (NP > 1) pass_bound(std::integral_constant<int, (NP > 1 ? 1 : 0)>{});
      if constexpr (NP > 2) pass_bound(std::integral_constant<int, (NP > 2 ? 2 : 0)>{});
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
    const float S = ldexpf(1.f, 30 - ex), invS = ldexpf(1.f, ex - 30);
    // the item's slice of the fp32 accumulator (input-shaped, this group's
    // 16 channels): cleared here for an item that takes atomics
    const __amdgpu_buffer_rsrc_t racc_img =
        make_rsrc(static_cast<unsigned char *>(bp.acc) + (size_t)cur.img * GX, img_bytes * GX);
    if (!fixed) {  // block-uniform
      typedef uint32_t u4 __attribute__((ext_vector_type(4)));
      const uint32_t npx = (uint32_t)p.H * (uint32_t)p.W;
      for (uint32_t t = threadIdx.x; t < npx * 4u; t += G::kThreads) {
        const uint32_t px = t >> 2, part = t & 3u;
        __builtin_amdgcn_raw_buffer_store_b128(
            u4{0u, 0u, 0u, 0u}, racc_img,
            (int)((px * pix_bytes + cur.g * (uint32_t)(CG * EB)) * GX + part * 16u), 0, 0);
      }
      __threadfence_block();
      __syncthreads();  // the slice is clear before any atomic adds into it
    }

    const uint32_t next = item + walk.stride;
    const bool more = next < end;  // block-uniform
    const Item nx = decode(more ? next : item);
    issue_window(nx, more);

#pragma unroll 1
    for (int pp = 0; pp < NP; ++pp) {
      bool live;
      const uint32_t pg = pass_pg(cur, pp, live);
      float m[P], gy[4];
      float2 offs[P];
      weights(std::integral_constant<int, 0>{}, m);
      unpack<DT, NWL>(rg[0], gy);
      // grad_output in the scatter's pair order
      const float gys[4] = {podd ? gy[2] : gy[0], podd ? gy[3] : gy[1], podd ? gy[0] : gy[2], podd ? gy[1] : gy[3]};
#pragma unroll
      for (int r = 0; r < P; ++r) {
        if constexpr (DT == DCN_F32)
          offs[r] = make_float2(__uint_as_float(rw[0][2 * r]), __uint_as_float(rw[0][2 * r + 1]));
        else
          offs[r] = make_float2(io::lo(rw[0][r]), io::hi(rw[0][r]));
      }

      // One round: every lane's point of slot r (its offset o2 and weight
      // mk, its window position (bx0, by0) before the offset), processed by
      // the whole quad; `owners` of the quad's lanes hold a point this round.
      // Returns the lane's own (gm, d/dx, d/dy).
      auto round = [&](float2 o2, float mk, int bx0, int by0, int owners) -> float3 {
        const float dx = s * o2.x, dy = s * o2.y;
        const bool nan_loc = (dx != dx) | (dy != dy);
        const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
        const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
        const float fx = floorf(cx), fy = floorf(cy);
        const float lx = cx - fx, ly = cy - fy;
        const float hx = 1.f - lx, hy = 1.f - ly;
        const int tx = bx0 + (int)fx;  // window coordinates of the top-left corner
        const int ty = by0 + (int)fy;
        // inside: the sample has a corner on the map (or on window pixels
        // past a map smaller than the window, which read and hold zeros)
        const bool inside = live && !nan_loc && (uint32_t)ty <= (uint32_t)LIM_Y && (uint32_t)tx <= (uint32_t)LIM_X;
        const uint32_t A = inside ? mad24((uint32_t)ty, (uint32_t)ROW, mul24((uint32_t)tx, PIXB)) : ZERO;
        const float wy1 = ly * mk, wy0 = mk - wy1;
        const float W1 = wy0 * lx, W0 = wy0 - W1;
        const float W3 = wy1 * lx, W2 = wy1 - W3;
        const float W0s = W0 * S, W1s = W1 * S, W2s = W2 * S, W3s = W3 * S;
        const uint32_t AS = inside ? A : SINK - GWIN;
        const bool gscat = !fixed && inside;  // global scatter (items off fixed point)
        const bool gs_any = __builtin_amdgcn_ballot_w64(gscat) != 0;  // wave-uniform
        float Gown[4] = {0.f, 0.f, 0.f, 0.f};  // the quad's corner sums of this lane's own point

        // Gather this lane's 4 channels of the four corners of the point of
        // lane O (input window; the corners 00, 01, 10, 11 in q[0..3],
        // q[4..7], ...).  A point's gather is issued before the previous
        // point's scatter: the two touch different windows, and the compiler
        // would not move reads across the LDS atomics by itself.
        auto gather = [&](auto o_tag, uint32_t (&q)[16]) {
          constexpr int O = decltype(o_tag)::value;
          const uint32_t src = add_bcast<O>(A, win_chunk);
          uint32_t q00[4], q01[4], q10[4], q11[4];
          lds_load_at<4>(src, q00);
          lds_load_at<4>(src + PIXB, q01);
          lds_load_at<4>(src + ROW, q10);
          lds_load_at<4>(src + ROW + PIXB, q11);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            q[c] = q00[c];
            q[4 + c] = q01[c];
            q[8 + c] = q10[c];
            q[12 + c] = q11[c];
          }
        };
        auto point = [&](auto o_tag, const uint32_t (&q)[16]) {
          constexpr int O = decltype(o_tag)::value;
          float Pc[4] = {0.f, 0.f, 0.f, 0.f};  // corners 00, 01, 10, 11
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            Pc[0] = fmaf(gy[c], __uint_as_float(q[c]), Pc[0]);
            Pc[1] = fmaf(gy[c], __uint_as_float(q[4 + c]), Pc[1]);
            Pc[2] = fmaf(gy[c], __uint_as_float(q[8 + c]), Pc[2]);
            Pc[3] = fmaf(gy[c], __uint_as_float(q[12 + c]), Pc[3]);
          }
          // Sums over the 16 channels: every lane of the quad gets them; the
          // owner keeps them (selects, no branch) for after the round.
          quad_sum4(Pc);
          const bool owner = sub == (uint32_t)O;
#pragma unroll
          for (int q = 0; q < 4; ++q) Gown[q] = owner ? Pc[q] : Gown[q];
          // Scatter m_k * w_corner * gy_c of this lane's 4 channels (no
          // branch: samples off the map add into the sink).
          if (fixed) {  // block-uniform
            const uint32_t d = add_bcast<O>(AS, gwin_chunk), d2 = d ^ 8u;  // the lane's first and second pair
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
            if (qbcast<O>((int)gscat)) {  // the whole quad follows its owner
              // fp32 accumulator offsets of the owner's four corners for this
              // lane's channels (out of range where a corner is off the map)
              const int yb = qbcast<O>(ty) - 1, xb = qbcast<O>(tx) - 1;
              const bool vy0 = (uint32_t)yb < (uint32_t)p.H, vy1 = (uint32_t)(yb + 1) < (uint32_t)p.H;
              const bool vx0 = (uint32_t)xb < (uint32_t)p.W, vx1 = (uint32_t)(xb + 1) < (uint32_t)p.W;
              const uint32_t a00 = (uint32_t)yb * row_bytes + (uint32_t)xb * pix_bytes + cur.chan;
              const uint32_t ga[4] = {(vy0 && vx0) ? a00 : kOutOfRange, (vy0 && vx1) ? a00 + pix_bytes : kOutOfRange,
                                      (vy1 && vx0) ? a00 + row_bytes : kOutOfRange,
                                      (vy1 && vx1) ? a00 + row_bytes + pix_bytes : kOutOfRange};
              const float wc[4] = {qbcast<O>(W0), qbcast<O>(W1), qbcast<O>(W2), qbcast<O>(W3)};
#pragma unroll
              for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                      wc[q] * gy[c], racc_img, (int)(ga[q] == kOutOfRange ? kOutOfRange : ga[q] * GX + 4u * c), 0, 0);
            }
          }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        uint32_t qa[16], qb[16];
        gather(I0{}, qa);
        if (owners > 1) gather(I1{}, qb);
        point(I0{}, qa);
        if (owners > 2) gather(I2{}, qa);
        if (owners > 1) point(I1{}, qb);
        if (owners > 3) gather(I3{}, qb);
        if (owners > 2) point(I2{}, qa);
        if (owners > 3) point(I3{}, qb);
        // gm, d/dx and d/dy of the own point (one-sided derivatives of the
        // bilinear form, linear in the corner sums); a lane without a point
        // this round returns values nobody stores.
        const float T = hx * Gown[0] + lx * Gown[1], Bt = hx * Gown[2] + lx * Gown[3];
        return nan_loc ? make_float3(qnan, qnan, qnan)
                       : make_float3(hy * T + ly * Bt, hy * (Gown[1] - Gown[0]) + ly * (Gown[3] - Gown[2]), Bt - T);
      };

      float3 res[P];
      res[2] = make_float3(0.f, 0.f, 0.f);
#pragma unroll
      for (int r = 0; r < ROUNDS; ++r)
        res[r] = round(offs[r], m[r], bx[r], by[r] + pp * (ST * TH), r < 2 ? 4 : 1);

      // Offset and mask gradients of the own slots (a NaN sampling location
      // makes its point's offset gradient and gm NaN).
      if (live) {
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
        float go[P][2];
#pragma unroll
        for (int r = 0; r < P; ++r) {
          go[r][0] = s * m[r] * res[r].y;
          go[r][1] = s * m[r] * res[r].z;
        }
        if constexpr (DT == DCN_F32) {
          typedef float f4 __attribute__((ext_vector_type(4)));
          typedef float f2 __attribute__((ext_vector_type(2)));
          const uint32_t orow = pg * (K * 8), mrow = pg * (K * 4);
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
          const uint32_t orow = pg * (K * 4), mrow = pg * (K * 2);
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
      // this pass's rows are no longer needed: shift the slots down and
      // request the next item's rows of this pass into the last
#pragma unroll
      for (int i = 0; i + 1 < NP; ++i) {
#pragma unroll
        for (int j = 0; j < NRW; ++j) rw[i][j] = rw[i + 1][j];
#pragma unroll
        for (int j = 0; j < P; ++j) rl[i][j] = rl[i + 1][j];
#pragma unroll
        for (int j = 0; j < NWL; ++j) rg[i][j] = rg[i + 1][j];
      }
      issue_rows(nx, pp, more, std::integral_constant<int, NP - 1>{});
    }

    __syncthreads();  // every scatter into the grad window (or the accumulator) is done
    // Write the item's grad_input slice: each lane one channel pair of a
    // window pixel (eight lanes per pixel), the window cleared as it is read.
    // Map pixels take the fixed-point sums (or, for an item on atomics, the
    // accumulator's values) rounded to the I/O dtype; border pixels and
    // pixels past the map are only cleared.
    {
      const __amdgpu_buffer_rsrc_t rgo_img = make_rsrc(static_cast<unsigned char *>(bp.grad_in) + cur.img, img_bytes);
      typedef __attribute__((address_space(3))) uint64_t L;
      const uint32_t pr = threadIdx.x & 7u;
      for (uint32_t t = threadIdx.x; t < (uint32_t)(SPAN_W * SPAN_H * 8); t += G::kThreads) {
        const uint32_t wp = t >> 3, y = wp / (uint32_t)SPAN_W, x = wp - y * (uint32_t)SPAN_W;
        L *slot = (L *)(size_t)(lbase + GWIN + wp * PIXB + pr * 8u);
        const int2 q = pair_sums(*slot);
        *slot = 0;
        const bool on_map = y - 1u < (uint32_t)p.H && x - 1u < (uint32_t)p.W;
        const uint32_t at = (y - 1u) * row_bytes + (x - 1u) * pix_bytes + cur.g * (uint32_t)(CG * EB) + pr * 2u * EB;
        float v0 = (float)q.x * invS, v1 = (float)q.y * invS;
        if (!fixed) {  // block-uniform
          if constexpr (DT == DCN_F32) continue;  // the accumulator is grad_input itself
          // (through the L2, where the atomics went)
          const auto a = __builtin_amdgcn_raw_buffer_load_b64(racc_img, on_map ? (int)(at * GX) : (int)kOutOfRange, 0, 1);
          v0 = __uint_as_float(a[0]);
          v1 = __uint_as_float(a[1]);
        }
        if constexpr (DT == DCN_F32) {
          typedef float f2 __attribute__((ext_vector_type(2)));
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint32_t __attribute__((ext_vector_type(2))), f2{v0, v1}),
                                                rgo_img, on_map ? (int)at : (int)kOutOfRange, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(io::pack(v0, v1), rgo_img, on_map ? (int)at : (int)kOutOfRange, 0, 0);
        }
      }
    }

    item = next;
    cur = nx;
  }
}

namespace {

template <int DT, bool SM, bool RC, int TW, int TH, int NP, int ST>
hipError_t launch_bwd_map(const BwdParams &p, const TileGeom &tg, hipStream_t s) {
  using G = BmGeom<TW, TH, NP, ST>;
  auto kern = dcn_bwd_map_kernel<DT, SM, RC, TW, TH, NP, ST>;
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

template <int TW, int TH, int NP, int ST>
hipError_t launch_map_dt(int dtype, int softmax, bool rc, const BwdParams &b, const TileGeom &tg, hipStream_t s) {
#define DCN_BM_LAUNCH(DT)                                                                      \
  return softmax ? (rc ? launch_bwd_map<DT, true, true, TW, TH, NP, ST>(b, tg, s)              \
                       : launch_bwd_map<DT, true, false, TW, TH, NP, ST>(b, tg, s))            \
                 : (rc ? launch_bwd_map<DT, false, true, TW, TH, NP, ST>(b, tg, s)             \
                       : launch_bwd_map<DT, false, false, TW, TH, NP, ST>(b, tg, s))
  switch (dtype) {
    case DCN_F32: DCN_BM_LAUNCH(DCN_F32);
    case DCN_F16: DCN_BM_LAUNCH(DCN_F16);
    case DCN_BF16: DCN_BM_LAUNCH(DCN_BF16);
    default: return hipErrorInvalidValue;
  }
#undef DCN_BM_LAUNCH
}

// Whole-map shapes: (TW, TH, NP, ST) with the output map within TW x NP*TH
// and the input map within ST*TW x ST*NP*TH; the first that holds the map at
// its stride is taken.
struct MapShape {
  int tw, th, np, st;
};
constexpr MapShape kMapShapes[] = {{12, 12, 1, 1}, {16, 16, 1, 1}, {24, 8, 3, 1}, {12, 12, 1, 2}};

int map_shape(const FwdParams &p) {
  if (p.KH != 3 || p.KW != 3 || p.SH != p.SW || p.DH != 1 || p.DW != 1) return -1;
  for (int i = 0; i < (int)(sizeof(kMapShapes) / sizeof(kMapShapes[0])); ++i) {
    const MapShape m = kMapShapes[i];
    if (p.SH == m.st && p.Wo <= m.tw && p.Ho <= m.th * m.np && p.W <= m.st * m.tw && p.H <= m.st * m.th * m.np)
      return i;
  }
  return -1;
}

}  // namespace

bool backward_map_applies(const FwdParams &p) {
  if (map_shape(p) < 0) return false;
  // every window row's offset relative to the image fits int32 (rows outside
  // the map are rejected by the image's buffer range), and so do the item's
  // fp32 accumulator offsets
  const int64_t row_bytes = (int64_t)p.W * p.C * 4;
  return ((int64_t)p.H + 2) * row_bytes < (int64_t(1) << 31);
}

hipError_t launch_backward_map(int dtype, int softmax, const BwdParams &b, hipStream_t s) {
  const FwdParams &p = b.f;
  if (!backward_map_applies(p)) return hipErrorNotSupported;
  const int64_t imgs = p.pg_total / ((int64_t)p.Ho * p.Wo * p.G);
  const int64_t items = imgs * p.G;
  if (items <= 0 || items >= (int64_t(1) << 31)) return hipErrorNotSupported;
  TileGeom tg{};
  tg.items = (uint32_t)items;
  tg.div_g = make_fast_div((uint32_t)p.G);
  switch (map_shape(p)) {
    case 0: return launch_map_dt<12, 12, 1, 1>(dtype, softmax, p.RC != 0, b, tg, s);
    case 1: return launch_map_dt<16, 16, 1, 1>(dtype, softmax, p.RC != 0, b, tg, s);
    case 2: return launch_map_dt<24, 8, 3, 1>(dtype, softmax, p.RC != 0, b, tg, s);
    case 3: return launch_map_dt<12, 12, 1, 2>(dtype, softmax, p.RC != 0, b, tg, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace dcn
