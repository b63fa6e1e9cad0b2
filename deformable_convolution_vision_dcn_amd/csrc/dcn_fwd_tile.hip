// dcn_fwd_tile.hip -- LDS-tiled gfx950 forward kernel of the DCN core for
// 3x3 kernel points (the InternImage configuration; wmrh.cn/news/61976,
// section 二 steps 2-4 and section 三), in fp32 also for the 8 points that
// DCNv4's remove_center leaves (pnsm.cn/news/2029644.html section 3.3).
//
// Why tiles: every bilinear sample reads four 16-channel corner slices at
// offset-driven addresses, 256 bytes per sample in fp32 against 59*4/9 bytes
// of compulsory traffic.  Served from the vector L1 those gathers top out
// near 60 B/clk per CU even when resident; LDS delivers about 105 B/clk for
// one lane-quad per 64-byte slice at an 80-byte pixel stride (measured on
// MI355X).  So each block stages the input window its samples can reach
// into LDS once and gathers from there.
//
// Block = 512 threads = 128 lane-quads; it owns one (image, TH x TW output
// tile, group).  Window = the tile's regular 3x3 footprint plus a halo of R
// pixels on each side for the learned offsets, zero-filled outside the map
// (so out-of-map corners read 0 from LDS like any other).  A sample whose
// corners leave the window (|s*offset| beyond the halo) is served from
// global memory instead, with the buffer range check supplying the zeros.
//
// Per pixel-group one quad: lane `sub` owns channels [4*sub, 4*sub+4) and
// computes the location, bilinear weights (modulation folded in) and LDS
// address of the kernel points k = 2 sub, 2 sub + 1 (and k = 8 for sub 0;
// in fp32 group pairs the second group's quad owns 2 sub + 1, 2 sub + 2 and,
// in lane 0, k = 0, see the row loads);
// DPP quad broadcasts hand them to the other three lanes, so no lane repeats
// another's address math.  Each lane then reads its 16-byte chunk of the four corners and does
// 4 FMAs per channel per point.  The softmax over the nine logits is a quad
// reduction (max, then sum of exponentials).
#include <algorithm>
#include <type_traits>

#include "dcn_device.hpp"
#include "quad_ops.hpp"

namespace dcn {


#ifndef DCN_TILE_WAVES
#define DCN_TILE_WAVES 4  // waves per SIMD the register budget must allow
#endif
#ifndef DCN_PIXB_F32
#define DCN_PIXB_F32 80   // LDS bytes per staged fp32 pixel slice (64 + pad)
#endif
#ifndef DCN_PIXB_16
#define DCN_PIXB_16 40    // LDS bytes per staged 16-bit pixel slice (32 + pad)
#endif

#ifndef DCN_TILE_MAXSPAN
#define DCN_TILE_MAXSPAN 1024
#endif
#ifndef DCN_PAIR_MAXSPAN
#define DCN_PAIR_MAXSPAN 1280
#endif

// GP = groups per work item.  GP = 2 stages the two neighbouring groups of a
// pixel together (one 128-byte line in fp32 instead of two half lines): half
// the window requests per pixel-group, offset and mask rows of both groups
// read by the same instructions, and a 1024-thread block per CU.
template <int GP>
constexpr int tile_max_span() { return GP == 1 ? DCN_TILE_MAXSPAN : DCN_PAIR_MAXSPAN; }

template <int DT, int GP>
constexpr int tile_pixel_stride() {
  return GP == 2 ? 2 * kGroupChannels * Io<DT>::kBytes : (DT == DCN_F32 ? DCN_PIXB_F32 : DCN_PIXB_16);
}

// UDIL > 0: stride 1 and dilation UDIL (1 or 2) on both axes, so the window
// geometry is a compile-time constant (no run-time multiplies on the
// per-point path); UDIL = 0: any stride and dilation.  RC: the centre
// point is removed (8 points, point k at grid index k + (k >= 4)): each lane
// owns two points, lane 0's third slot stays empty, two rounds instead of
// three.
template <int DT, bool SOFTMAX, int TH, int TW, int R, int UDIL, int GP, bool RC>
__global__ void __launch_bounds__(512 * GP, DCN_TILE_WAVES) dcn_fwd_tile_kernel(FwdParams p, TileGeom tg) {
  using io = Io<DT>;
  constexpr int CG = kGroupChannels;
  constexpr int CPL = 4;                           // channels per lane
  constexpr int NW = CPL * io::kBytes / 4;         // words per lane per corner
  constexpr int LANE_BYTES = CPL * io::kBytes;
  constexpr int THREADS = 512 * GP;
  constexpr int PIXB = tile_pixel_stride<DT, GP>();
  constexpr int GBYTES = CG * io::kBytes;          // one group of one pixel
  constexpr int QUADS = THREADS / 4;
  constexpr int PIXPP = QUADS / GP;                // output pixels per pass
  constexpr int PASSES = TH * TW / PIXPP;
  constexpr int LPP = 4 * GP;                      // lanes per staged window pixel
  constexpr int WPIX = THREADS / LPP;              // window pixels per slice
  constexpr int MAXPQ = (tile_max_span<GP>() + WPIX - 1) / WPIX;  // slices per lane
  constexpr int K = RC ? 8 : 9;
  // fp32 group pairs of nine points: the quads of the pair's two groups split
  // its 144-byte offset row at the middle chunk (see the row loads).
  constexpr bool SPLIT = DT == DCN_F32 && GP == 2 && !RC;
  static_assert(PASSES == 1 || PASSES == 2, "one or two passes per item");
  static_assert(PIXB % LANE_BYTES == 0 && PIXB % 8 == 0 && PIXB >= GP * 4 * LANE_BYTES, "pixel stride");
  static_assert(GP == 1 || GP == 2, "one or two groups per item");

  extern __shared__ __align__(16) unsigned char tile[];

  // Quad -> (output pixel of the pass, group of the item).  With two groups
  // the four quads of a 16-lane LDS phase are two pixels x two groups, so
  // their 64-byte corner reads fall in two bank halves per group.
  const uint32_t quad = threadIdx.x >> 2, sub = threadIdx.x & 3;
  const uint32_t gsel = GP == 1 ? 0u : (quad >> 1) & 1u;
  const uint32_t pix = GP == 1 ? quad : ((quad >> 2) << 1) | (quad & 1u);
  const uint32_t wlane = threadIdx.x % LPP;        // 16-byte chunk of a window pixel
  const uint32_t pix_bytes = (uint32_t)p.C * io::kBytes;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  // Rows and outputs go through buffer instructions too: with 32-bit offsets
  // the address unit handles them several times faster than 64-bit global
  // addresses when a wave touches many cache lines.
  const __amdgpu_buffer_rsrc_t roff = make_rsrc(p.offset, p.off_bytes);
  const __amdgpu_buffer_rsrc_t rmask = make_rsrc(p.mask, p.mask_bytes);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(p.output, p.out_bytes);
  constexpr bool UNIT = UDIL > 0;
  constexpr int USPAN = TW + 2 * R + 1 + 2 * UDIL;  // window edge at stride 1, dilation UDIL
  const int span_w = UNIT ? USPAN : tg.span_w;
  const int span_h = UNIT ? (TH + 2 * R + 1 + 2 * UDIL) : tg.span_h;
  const int span = span_h * span_w;
  const int row_lds = span_w * PIXB;
  const int zero_base = span * PIXB;
  const int lim_y = span_h - 2, lim_x = span_w - 2;
  const int SW = UNIT ? 1 : p.SW, SH = UNIT ? 1 : p.SH;
  const int DW = UNIT ? UDIL : p.DW, DH = UNIT ? UDIL : p.DH;
  const float s = p.scale;

  // Window slots at unit stride.  A lane stages the same window pixels of
  // every item: main slice u holds window rows [u RPS, u RPS + RPS) of
  // columns [0, CW), the last slices the rows below and the columns right of
  // that block.  So the per-item address work is one uniform base plus one
  // column check per lane; rows outside the map fall out of the image's
  // buffer range (negative or past its last byte) and read zero.
  constexpr int CW = USPAN > 32 ? 32 : USPAN;
  constexpr int RPS = WPIX / CW;
  constexpr int NM = USPAN / RPS;
  constexpr int REM_A = (USPAN - NM * RPS) * CW, REM_B = (USPAN - CW) * USPAN;
  constexpr int NR = (REM_A + REM_B + WPIX - 1) / WPIX;  // remainder slices
  constexpr int WSL = UNIT ? NM + NR : MAXPQ;            // register slices of a window
  static_assert(!UNIT || (NR >= 1 && NM + NR <= MAXPQ), "window slot mapping");
  const uint32_t slot = threadIdx.x / LPP;
  const uint32_t m_col = slot % CW;
  const bool m_live = slot < (uint32_t)(RPS * CW);
  // remainder pixel rs = rho * WPIX + slot of remainder slice rho (the
  // arrays keep one element where the run-time geometry has no remainder)
  constexpr int NRA = NR > 0 ? NR : 1;
  uint32_t r_y[NRA], r_x[NRA];
  bool r_live[NRA];
#pragma unroll
  for (int rho = 0; rho < NR; ++rho) {
    const uint32_t rs = (uint32_t)rho * WPIX + slot;
    r_y[rho] = 0;
    r_x[rho] = 0;
    if (rs < (uint32_t)REM_A) {
      r_y[rho] = NM * RPS + rs / CW;
      r_x[rho] = rs % CW;
    } else if constexpr (USPAN > CW) {
      r_y[rho] = (rs - REM_A) / (USPAN - CW);
      r_x[rho] = CW + (rs - REM_A) % (USPAN - CW);
    }
    r_live[rho] = rs < (uint32_t)(REM_A + REM_B);
  }
  const uint32_t m_lane = (slot / CW) * row_bytes + m_col * pix_bytes + wlane * LANE_BYTES;
  uint32_t r_lane[NRA];
#pragma unroll
  for (int rho = 0; rho < NR; ++rho) r_lane[rho] = r_y[rho] * row_bytes + r_x[rho] * pix_bytes + wlane * LANE_BYTES;
  const uint32_t img_bytes = (uint32_t)p.H * row_bytes;

  // Window coordinates of the kernel point of each own slot before its
  // offset, for pass 0 (pass 1 adds PIXPP / TW output rows), packed as three
  // 10-bit fields (every coordinate is below the span, at most 1023).  The
  // output pixel of the quad is (pix / TW, pix % TW) within its pass; slot r
  // holds k = 2 sub + r (r < 2) or k = 8 (no point with RC), at grid index q;
  // with SPLIT the second group's quad holds k = 2 sub + r + 1 and k = 0.
  const int kshift = SPLIT ? (int)gsel : 0;
  uint32_t bxp = 0, byp = 0;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int k = r < 2 ? 2 * (int)sub + r + kshift : (kshift ? 0 : 8);
    const int q = RC ? (r < 2 ? k + (k >= 4) : 4) : k;
    const int i = q / 3, j = q - 3 * (q / 3);
    bxp |= (uint32_t)((int)(pix % TW) * SW + R + j * DW) << (10 * r);
    byp |= (uint32_t)((int)(pix / TW) * SH + R + i * DH) << (10 * r);
  }
  typedef __attribute__((address_space(3))) unsigned char lds_byte;
  const uint32_t lane_chunk = (uint32_t)(size_t)(lds_byte *)tile + gsel * GBYTES + sub * LANE_BYTES;

  // A zero block after the window: samples served from global memory (and
  // NaN locations) read their main-path corners here, contributing w * 0.
  // Written once; the first barrier of the item loop orders it.
  for (int z = (int)threadIdx.x * 8; z < row_lds + 2 * PIXB; z += THREADS * 8)
    *reinterpret_cast<uint2 *>(tile + zero_base + z) = make_uint2(0, 0);

  // Work item -> (n, tile, first group g); g varies fastest so the items that
  // share an input window's cache lines (neighbouring groups) run close in
  // time.  chan: this quad's group and lane chunk (the fix-up gathers);
  // wchan: this lane's chunk of a staged window pixel.
  struct Item {
    uint32_t g, n, img, chan, wchan;
    int r0, c0, Y0, X0;
  };
  auto decode = [&](uint32_t it) {
    Item I;
    const uint32_t t = fast_div(it, tg.div_g);
    I.g = (it - t * ((uint32_t)p.G / GP)) * GP;
    I.n = fast_div(t, tg.div_tiles);
    const uint32_t tile_id = t - I.n * (uint32_t)tg.tiles_per_img;
    const uint32_t tyi = fast_div(tile_id, tg.div_tiles_x);
    const uint32_t txi = tile_id - tyi * (uint32_t)tg.tiles_x;
    I.r0 = (int)tyi * TH;
    I.c0 = (int)txi * TW;
    I.Y0 = I.r0 * SH - p.PH - R;  // window origin in input coordinates
    I.X0 = I.c0 * SW - p.PW - R;
    I.img = I.n * (uint32_t)p.H * row_bytes;
    I.chan = ((I.g + gsel) * CG + sub * CPL) * io::kBytes;
    I.wchan = I.g * GBYTES + wlane * LANE_BYTES;
    return I;
  };

  // Window slices of an item, LPP lanes per pixel: requested into registers
  // while the previous item computes, written to LDS when it is done.
  uint32_t win[WSL][NW];
  // Issued on every path (an item that does not exist loads nothing: every
  // offset out of range), so that the compiler's count of outstanding loads
  // stays exact and no wait covers a prefetch before it is needed.
  auto issue_window = [&](const Item &I, bool valid) {
    if constexpr (UNIT) {
      const __amdgpu_buffer_rsrc_t rimg = make_rsrc(static_cast<const unsigned char *>(p.input) + I.img, img_bytes);
      const uint32_t base = (uint32_t)I.Y0 * row_bytes + (uint32_t)I.X0 * pix_bytes + I.g * GBYTES;  // mod 2^32
      const uint32_t m_off = valid && m_live && (uint32_t)(I.X0 + (int)m_col) < (uint32_t)p.W ? base + m_lane : kOutOfRange;
#pragma unroll
      for (int u = 0; u < NM; ++u) buffer_load_words<NW>(rimg, m_off + (uint32_t)(u * RPS) * row_bytes, win[u]);
#pragma unroll
      for (int rho = 0; rho < NR; ++rho) {
        const uint32_t r_off = valid && r_live[rho] && (uint32_t)(I.X0 + (int)r_x[rho]) < (uint32_t)p.W
                                   ? base + r_lane[rho] : kOutOfRange;
        buffer_load_words<NW>(rimg, r_off, win[NM + rho]);
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < MAXPQ; ++u) {
      const int idx = (int)(threadIdx.x / LPP) + u * WPIX;
      uint32_t offb = kOutOfRange;
      if (valid && idx < span) {
        const int sy = UNIT ? idx / USPAN : (int)fast_div((uint32_t)idx, tg.div_span_w);
        const int sx = idx - sy * span_w;
        const int gy = I.Y0 + sy, gx = I.X0 + sx;
        if ((uint32_t)gy < (uint32_t)p.H && (uint32_t)gx < (uint32_t)p.W)
          offb = I.img + (uint32_t)gy * row_bytes + (uint32_t)gx * pix_bytes + I.wchan;
      }
      buffer_load_words<NW>(rin, offb, win[u]);
    }
  };
  auto store_window = [&]() {
    if constexpr (UNIT) {
      const uint32_t m_lds = (slot / CW) * row_lds + m_col * PIXB + wlane * LANE_BYTES;
#pragma unroll
      for (int u = 0; u < NM; ++u)
        if (m_live) lds_store<NW>(tile + m_lds + u * RPS * row_lds, win[u]);
#pragma unroll
      for (int rho = 0; rho < NR; ++rho)
        if (r_live[rho]) lds_store<NW>(tile + r_y[rho] * row_lds + r_x[rho] * PIXB + wlane * LANE_BYTES, win[NM + rho]);
      return;
    }
#pragma unroll
    for (int u = 0; u < MAXPQ; ++u) {
      const int idx = (int)(threadIdx.x / LPP) + u * WPIX;
      if (idx < span) lds_store<NW>(tile + idx * PIXB + wlane * LANE_BYTES, win[u]);
    }
  };

  // Own points' offsets and logits of both passes: the quad owns output
  // pixel pp = ps*PIXPP + pix of the tile, group g + gsel; lane `sub` owns the
  // points k = 2 sub, 2 sub + 1 (slots 0, 1) and lane 0 also k = 8 (slot 2)
  // (SPLIT below shifts the second group's by one), so a quad reads its
  // pixel-group's offset and mask rows contiguously.
  // The rows are kept as loaded (raw words) and decoded where they are used:
  // any arithmetic on them here would make the wave wait for the load at
  // once.  Every lane loads every slot (a dead quad reads row 0), so the
  // loads carry no conditions either.
  //   fp32:   rw = x, y of k = 2 sub; x, y of 2 sub + 1; x, y of k = 8;
  //           rl = logits of 2 sub, 2 sub + 1, 8.
  //   16-bit: rw = (x, y) words of 2 sub, 2 sub + 1, 8; rl = logit halves.
  //   SPLIT:  rw = x, y of the quad's points 2 sub + gsel, 2 sub + gsel + 1
  //           and of its slot-2 point (8 or 0); rl = the group's logits
  //           2 sub, 2 sub + 1, 2 sub + 2.
  // SPLIT: a pixel's pair of offset rows is 144 contiguous bytes, nine
  // 16-byte chunks.  The first group's quad reads chunks 0-3 (its points
  // 0-7), the second group's quad chunks 5-8 (its points 1-8), and chunk 4
  // holds the first group's point 8 and the second's point 0, one line for
  // every pixel; the logits take one 12-byte load per lane.  Per wave that
  // is three row loads touching about 4.6 lines per pixel instead of four
  // touching about 6.5 (11 % fewer vector-memory reads per launch at the
  // stage-1 shape).  Lane 0 of the first group takes its ninth logit from
  // lane 3.
  constexpr int NRW = DT == DCN_F32 ? 6 : 3;
  uint32_t rw[PASSES][NRW], rl[PASSES][3];
  auto load_rows = [&](uint32_t pg, uint32_t (&w)[NRW], uint32_t (&l)[3]) {
    if constexpr (SPLIT) {
      const uint32_t orow = pg * 72u, mrow = pg * 36u;
      const auto o = __builtin_amdgcn_raw_buffer_load_b128(roff, (int)(orow + 16 * sub + 8 * gsel), 0, 0);
      const auto o8 = __builtin_amdgcn_raw_buffer_load_b64(roff, (int)(gsel ? orow : orow + 64), 0, 0);
      const auto lg = __builtin_amdgcn_raw_buffer_load_b96(rmask, (int)(mrow + 8 * sub), 0, 0);
      w[0] = o[0];
      w[1] = o[1];
      w[2] = o[2];
      w[3] = o[3];
      w[4] = o8[0];
      w[5] = o8[1];
      l[0] = lg[0];
      l[1] = lg[1];
      l[2] = lg[2];
    } else if constexpr (DT == DCN_F32) {
      const uint32_t orow = pg * (K * 8), mrow = pg * (K * 4);
      const auto o = __builtin_amdgcn_raw_buffer_load_b128(roff, (int)(orow + 16 * sub), 0, 0);
      const auto lg = __builtin_amdgcn_raw_buffer_load_b64(rmask, (int)(mrow + 8 * sub), 0, 0);
      w[0] = o[0];
      w[1] = o[1];
      w[2] = o[2];
      w[3] = o[3];
      l[0] = lg[0];
      l[1] = lg[1];
      if constexpr (RC) {
        w[4] = w[5] = l[2] = 0u;
      } else {
        const auto o8 = __builtin_amdgcn_raw_buffer_load_b64(roff, (int)(orow + 64), 0, 0);
        w[4] = o8[0];
        w[5] = o8[1];
        l[2] = __builtin_amdgcn_raw_buffer_load_b32(rmask, (int)(mrow + 32), 0, 0);
      }
    } else {
      const uint32_t orow = pg * (K * 4), mrow = pg * (K * 2);
      const auto o = __builtin_amdgcn_raw_buffer_load_b64(roff, (int)(orow + 8 * sub), 0, 0);
      w[0] = o[0];
      w[1] = o[1];
      if constexpr (RC) {  // 16-byte mask rows: the lane's two logits in one word
        const uint32_t lw = __builtin_amdgcn_raw_buffer_load_b32(rmask, (int)(mrow + 4 * sub), 0, 0);
        l[0] = lw & 0xffffu;
        l[1] = lw >> 16;
        w[2] = l[2] = 0u;
      } else {
        w[2] = __builtin_amdgcn_raw_buffer_load_b32(roff, (int)(orow + 32), 0, 0);
        l[0] = __builtin_amdgcn_raw_buffer_load_b16(rmask, (int)(mrow + 4 * sub), 0, 0);
        l[1] = __builtin_amdgcn_raw_buffer_load_b16(rmask, (int)(mrow + 4 * sub + 2), 0, 0);
        l[2] = __builtin_amdgcn_raw_buffer_load_b16(rmask, (int)(mrow + 16), 0, 0);
      }
    }
  };
  auto issue_pgdata = [&](const Item &I, auto ps_tag) {
    constexpr int ps = decltype(ps_tag)::value;
    const int pp = ps * PIXPP + (int)pix;
    const int ho = I.r0 + pp / TW, wo = I.c0 + pp % TW;
    const bool live = ho < p.Ho && wo < p.Wo;
    const uint32_t pg = live ? (((I.n * (uint32_t)p.Ho + ho) * (uint32_t)p.Wo + wo) * (uint32_t)p.G) + I.g + gsel : 0u;
    load_rows(pg, rw[ps], rl[ps]);
  };
  // Decoded offsets (x, y) and logits of three slots.
  auto decode_rows = [&](const uint32_t (&w)[NRW], const uint32_t (&l)[3], float2 (&o)[3], float (&lg)[3]) {
    if constexpr (SPLIT) {
#pragma unroll
      for (int r = 0; r < 3; ++r) o[r] = make_float2(__uint_as_float(w[2 * r]), __uint_as_float(w[2 * r + 1]));
      const uint32_t l8 = (uint32_t)qbcast<3>((int)l[2]);  // the first group's logit 8 (all four lanes live)
      lg[0] = __uint_as_float(gsel ? l[1] : l[0]);
      lg[1] = __uint_as_float(gsel ? l[2] : l[1]);
      lg[2] = __uint_as_float(gsel ? l[0] : l8);
    } else if constexpr (DT == DCN_F32) {
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        o[r] = make_float2(__uint_as_float(w[2 * r]), __uint_as_float(w[2 * r + 1]));
        lg[r] = __uint_as_float(l[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        o[r] = make_float2(Io<DT>::lo(w[r]), Io<DT>::hi(w[r]));
        lg[r] = Io<DT>::lo(l[r]);
      }
    }
  };

  const XcdWalk walk = xcd_walk(blockIdx.x, gridDim.x, tg.items);
  const uint32_t end = walk.end;
  uint32_t item = walk.first;
  Item cur = decode(item < end ? item : 0);
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if (item < end) {
    issue_window(cur, true);
    issue_pgdata(cur, P0{});
    if constexpr (PASSES == 2) issue_pgdata(cur, P1{});
  }

  while (item < end) {
    __syncthreads();  // every wave is done reading the previous window
    store_window();
    __syncthreads();  // the window is in LDS

    // The next item's window is requested now and lands during this item's
    // passes; its per-pass offsets/logits are requested as soon as this
    // item's pass has consumed the registers they go to.
    const uint32_t next = item + walk.stride;
    const bool more = next < end;  // block-uniform
    const Item nx = decode(more ? next : item);
    issue_window(nx, more);

    auto pass = [&](auto ps_tag) {
      constexpr int ps = decltype(ps_tag)::value;
      const int pp = ps * PIXPP + (int)pix;
      const int ho = cur.r0 + pp / TW, wo = cur.c0 + pp % TW;
      if (ho >= p.Ho || wo >= p.Wo) return;  // whole quad leaves together
      const uint32_t pg = (((cur.n * (uint32_t)p.Ho + ho) * (uint32_t)p.Wo + wo) * (uint32_t)p.G) + cur.g + gsel;

      // Offsets and modulation weights of the three slots (softmax over the
      // quad's nine logits for DCNv3, the raw mask for DCNv4).
      float2 offs[3];
      float lgs[3], m[3];
      decode_rows(rw[ps], rl[ps], offs, lgs);
      if (RC || sub != 0) lgs[2] = SOFTMAX ? -INFINITY : 0.f;  // slot 2 is lane 0's point 8 (or 0) only
      if constexpr (SOFTMAX) {
        const float mx = quad_max(fmaxf(fmaxf(lgs[0], lgs[1]), lgs[2]));
        float e[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) e[r] = (r < 2 || (!RC && sub == 0)) ? __expf(lgs[r] - mx) : 0.f;
        const float inv = __builtin_amdgcn_rcpf(quad_sum(e[0] + e[1] + e[2]));
#pragma unroll
        for (int r = 0; r < 3; ++r) m[r] = e[r] * inv;
      } else {
#pragma unroll
        for (int r = 0; r < 3; ++r) m[r] = lgs[r];
      }

      float acc[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = 0.f;

      // Round r: every lane prepares its own point of slot r (location,
      // weights with the modulation folded in, window address), then the
      // quad consumes the round's points one owner at a time, the owner's
      // address and weights reaching the other lanes as DPP operands.
      const int by_pass = ps * (PIXPP / TW) * SH;
      auto round = [&](auto r_tag) {
        constexpr int r = decltype(r_tag)::value;
        const float2 o2 = offs[r];
        const float mk = m[r];
        const float dx = s * o2.x, dy = s * o2.y;
        const bool nan_loc = (dx != dx) | (dy != dy);
        const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
        const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
        const float fx = floorf(cx), fy = floorf(cy);
        const float lx = cx - fx, ly = cy - fy;
        // window coordinates of the top-left corner
        const int tx = (int)((bxp >> (10 * r)) & 1023u) + (int)fx;
        const int ty = (int)((byp >> (10 * r)) & 1023u) + by_pass + (int)fy;
        const float mkk = nan_loc ? __builtin_nanf("") : mk;  // NaN location: NaN weights
        const float wy1 = ly * mkk, wy0 = mkk - wy1;
        const float W1 = wy0 * lx, W0 = wy0 - W1;
        const float W3 = wy1 * lx, W2 = wy1 - W3;
        const bool inside = !nan_loc && (uint32_t)ty <= (uint32_t)lim_y && (uint32_t)tx <= (uint32_t)lim_x;
        const uint32_t A = inside ? mad24((uint32_t)ty, (uint32_t)row_lds, mul24((uint32_t)tx, PIXB)) : (uint32_t)zero_base;
        // outside the window: the global fix-up (whose buffer range check
        // reads zeros for corners off the map, so a sample that misses the
        // map entirely costs a rare gather instead of a test per round)
        const bool fb = !inside && !nan_loc;

        // Main path, no branches: gather the round's corners from LDS.
        auto point = [&](auto o_tag) {
          constexpr int O = decltype(o_tag)::value;
          uint32_t q00[NW], q01[NW], q10[NW], q11[NW];
          const uint32_t src = add_bcast<O>(A, lane_chunk);
          lds_load_at<NW>(src, q00);
          lds_load_at<NW>(src + PIXB, q01);
          lds_load_at<NW>(src + row_lds, q10);
          lds_load_at<NW>(src + row_lds + PIXB, q11);
          float v00[CPL], v01[CPL], v10[CPL], v11[CPL];
          unpack<DT, NW>(q00, v00);
          unpack<DT, NW>(q01, v01);
          unpack<DT, NW>(q10, v10);
          unpack<DT, NW>(q11, v11);
          fma4_bcast<O>(acc, W0, v00);
          fma4_bcast<O>(acc, W1, v01);
          fma4_bcast<O>(acc, W2, v10);
          fma4_bcast<O>(acc, W3, v11);
        };
        // Fix-up for points whose corners left the window: global gathers,
        // the buffer range check reading 0 for corners outside the map.
        auto fixup = [&](auto o_tag) {
          constexpr int O = decltype(o_tag)::value;
          if (!qbcast<O>((int)fb)) return;
          const int yb = qbcast<O>(ty) + cur.Y0, xb = qbcast<O>(tx) + cur.X0;
          const bool vy0 = (uint32_t)yb < (uint32_t)p.H, vy1 = (uint32_t)(yb + 1) < (uint32_t)p.H;
          const bool vx0 = (uint32_t)xb < (uint32_t)p.W, vx1 = (uint32_t)(xb + 1) < (uint32_t)p.W;
          const uint32_t a00 = cur.img + (uint32_t)yb * row_bytes + (uint32_t)xb * pix_bytes + cur.chan;
          uint32_t q00[NW], q01[NW], q10[NW], q11[NW];
          buffer_load_words<NW>(rin, (vy0 && vx0) ? a00 : kOutOfRange, q00);
          buffer_load_words<NW>(rin, (vy0 && vx1) ? a00 + pix_bytes : kOutOfRange, q01);
          buffer_load_words<NW>(rin, (vy1 && vx0) ? a00 + row_bytes : kOutOfRange, q10);
          buffer_load_words<NW>(rin, (vy1 && vx1) ? a00 + row_bytes + pix_bytes : kOutOfRange, q11);
          float v00[CPL], v01[CPL], v10[CPL], v11[CPL];
          unpack<DT, NW>(q00, v00);
          unpack<DT, NW>(q01, v01);
          unpack<DT, NW>(q10, v10);
          unpack<DT, NW>(q11, v11);
          fma4_bcast<O>(acc, W0, v00);
          fma4_bcast<O>(acc, W1, v01);
          fma4_bcast<O>(acc, W2, v10);
          fma4_bcast<O>(acc, W3, v11);
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        point(I0{});
        if constexpr (r < 2) {  // the last round holds only lane 0's slot-2 point
          point(I1{});
          point(I2{});
          point(I3{});
        }
        if (__builtin_amdgcn_ballot_w64(fb) != 0) {  // a quad of the wave left its window
          fixup(I0{});
          if constexpr (r < 2) {
            fixup(I1{});
            fixup(I2{});
            fixup(I3{});
          }
        }
      };
      round(std::integral_constant<int, 0>{});
      round(std::integral_constant<int, 1>{});
      if constexpr (!RC) round(std::integral_constant<int, 2>{});
      uint32_t outw[NW];
      pack_words<DT, CPL>(acc, outw);
      // Outputs are not read again here: stored non-temporal, so they do not
      // displace window and row lines from the L2.
      buffer_store_words_aux<NW, kNonTemporal>(rout, (pg * CG + sub * CPL) * io::kBytes, outw);
    };
    // Wave priority by progress: waves still in pass 0 issue ahead of waves
    // in pass 1, and waves done with the item yield, so the block reaches
    // its next barrier with less spread between its fastest and slowest
    // waves (all of them wait there for the slowest).
    __builtin_amdgcn_s_setprio(2);
    pass(P0{});
    __builtin_amdgcn_s_setprio(1);
    issue_pgdata(nx, P0{});  // unconditional (see issue_window)
    if constexpr (PASSES == 2) {
      pass(P1{});
      __builtin_amdgcn_s_setprio(0);
      issue_pgdata(nx, P1{});
    } else {
      __builtin_amdgcn_s_setprio(0);
    }

    item = next;
    cur = nx;
  }
}

namespace {

#ifndef DCN_TILE_HALO
#define DCN_TILE_HALO 6
#endif
#ifndef DCN_PAIR_HALO
#define DCN_PAIR_HALO 8
#endif
constexpr int kTileH = 16, kTileW = 16;
// Halo and LDS budget per variant: one group per item runs two 512-thread
// blocks per CU (80 KB each); two groups per item one 1024-thread block
// (up to the 160 KB of a CU).
template <int GP>
constexpr int tile_halo() { return GP == 1 ? DCN_TILE_HALO : DCN_PAIR_HALO; }
template <int GP>
constexpr int tile_lds_limit() { return GP == 1 ? 80 * 1024 : 160 * 1024; }
// One group per item at stride or dilation above 1: the halo taken when the
// default one overflows the window budget (dilation 2: a 31x31 window).
constexpr int kTileHaloSmall = 5;
// Two groups per item at other strides and dilations: 8-row output tiles and
// a halo of 4 (3 where 4 overflows; stride 2 at dilation 1 takes a 26 x 42
// window, 145 KB).
constexpr int kPairStridedTH = 8;
constexpr int kPairHaloStrided = 4;

size_t tile_lds_bytes(const TileGeom &tg, int pixb) {
  return ((size_t)tg.span_h * tg.span_w + tg.span_w + 2) * pixb;  // window + zero block
}

template <int DT, bool SM, int UDIL, int GP, bool RC, int HALO = tile_halo<GP>(), int TH = kTileH>
hipError_t launch_tile(const FwdParams &p, const TileGeom &tg, hipStream_t s) {
  auto kern = dcn_fwd_tile_kernel<DT, SM, TH, kTileW, HALO, UDIL, GP, RC>;
  const size_t lds = tile_lds_bytes(tg, tile_pixel_stride<DT, GP>());
  // Set on every launch: the limit is per device and setting it is idempotent.
  const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, tile_lds_limit<GP>());
  if (attr != hipSuccess) return attr;
  // Persistent blocks, 1024 threads per CU; each XCD walks one contiguous
  // range of items.
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const uint32_t blocks = std::min<uint32_t>(tg.items, (2u / GP) * (uint32_t)cus);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(512 * GP), lds, s, p, tg);
  return hipGetLastError();
}

// udil: the compile-time geometry's dilation (1 or 2 at stride 1), 0 for
// any other stride/dilation (one group per item only).
template <int DT, int GP, bool RC>
hipError_t launch_tile_dt(int softmax, int udil, int halo, const FwdParams &p, const TileGeom &tg, hipStream_t s) {
  constexpr int H2 = tile_halo<GP>() - 1;  // dilation 2: the same window edge as dilation 1
  if (udil == 1)
    return softmax ? launch_tile<DT, true, 1, GP, RC>(p, tg, s) : launch_tile<DT, false, 1, GP, RC>(p, tg, s);
  if (udil == 2)
    return softmax ? launch_tile<DT, true, 2, GP, RC, H2>(p, tg, s) : launch_tile<DT, false, 2, GP, RC, H2>(p, tg, s);
  if constexpr (GP == 2) {
    // other strides and dilations: 8 x 16 output tiles (one pass of 128
    // pixels x 2 groups), so that the strided window fits
    if (halo == kPairHaloStrided)
      return softmax ? launch_tile<DT, true, 0, GP, RC, kPairHaloStrided, kPairStridedTH>(p, tg, s)
                     : launch_tile<DT, false, 0, GP, RC, kPairHaloStrided, kPairStridedTH>(p, tg, s);
    if (halo == kPairHaloStrided - 1)
      return softmax ? launch_tile<DT, true, 0, GP, RC, kPairHaloStrided - 1, kPairStridedTH>(p, tg, s)
                     : launch_tile<DT, false, 0, GP, RC, kPairHaloStrided - 1, kPairStridedTH>(p, tg, s);
    return hipErrorNotSupported;
  } else {
    if (halo == kTileHaloSmall)
      return softmax ? launch_tile<DT, true, 0, GP, RC, kTileHaloSmall>(p, tg, s)
                     : launch_tile<DT, false, 0, GP, RC, kTileHaloSmall>(p, tg, s);
    return softmax ? launch_tile<DT, true, 0, GP, RC>(p, tg, s) : launch_tile<DT, false, 0, GP, RC>(p, tg, s);
  }
}

// Window geometry and work items for GP groups per item; false when the
// problem does not fit this variant.
template <int GP>
bool tile_geometry(int dtype, const FwdParams &p, TileGeom &tg, int halo, int th = kTileH) {
  if (p.G % GP != 0) return false;
  tg = TileGeom{};
  tg.span_h = (th - 1) * p.SH + 2 * p.DH + 2 * halo + 2;
  tg.span_w = (kTileW - 1) * p.SW + 2 * p.DW + 2 * halo + 2;
  const int pixb = dtype == DCN_F32 ? tile_pixel_stride<DCN_F32, GP>() : tile_pixel_stride<DCN_F16, GP>();
  if (tile_lds_bytes(tg, pixb) > (size_t)tile_lds_limit<GP>()) return false;
  if (tg.span_h * tg.span_w > tile_max_span<GP>()) return false;
  // At unit stride the window rows above and below the map are rejected by
  // the buffer range of their image, which needs the byte offset of every
  // window row relative to the image (rows -pad - halo - 1 to
  // H + pad + halo + 1) to fit int32.
  const bool unit = p.SH == 1 && p.SW == 1 && p.DH == p.DW && (p.DH == 1 || p.DH == 2);
  const int64_t row_bytes = (int64_t)p.W * p.C * (dtype == DCN_F32 ? 4 : 2);
  if (unit && ((int64_t)p.H + p.PH + tg.span_h + 1) * row_bytes >= (int64_t(1) << 31)) return false;
  const int tiles_y = (p.Ho + th - 1) / th;
  tg.tiles_x = (p.Wo + kTileW - 1) / kTileW;
  tg.tiles_per_img = tiles_y * tg.tiles_x;
  const int64_t imgs = p.pg_total / ((int64_t)p.Ho * p.Wo * p.G);
  const int64_t items = imgs * tg.tiles_per_img * (p.G / GP);
  if (items <= 0 || items >= (int64_t(1) << 31)) return false;
  tg.div_g = make_fast_div((uint32_t)(p.G / GP));
  tg.div_tiles = make_fast_div((uint32_t)tg.tiles_per_img);
  tg.div_tiles_x = make_fast_div((uint32_t)tg.tiles_x);
  tg.div_span_w = make_fast_div((uint32_t)tg.span_w);
  tg.items = (uint32_t)items;
  return true;
}

template <int GP>
hipError_t launch_tile_gp(int dtype, int softmax, const FwdParams &p, hipStream_t s) {
  TileGeom tg;
  // Stride 1 at dilation 1 or 2 (equal on both axes) runs the compile-time
  // geometry; dilation 2 takes a halo one smaller, so the window keeps its
  // edge.  Other strides and dilations run the general one-group variant.
  const int udil = (p.SH == 1 && p.SW == 1 && p.DH == p.DW && (p.DH == 1 || p.DH == 2)) ? p.DH : 0;
  int halo = tile_halo<GP>() - (udil == 2 ? 1 : 0);
  if (GP == 2 && udil == 0) {  // strided or unevenly dilated windows: 8-row tiles
    halo = kPairHaloStrided;
    if (!tile_geometry<GP>(dtype, p, tg, halo, kPairStridedTH)) {
      halo = kPairHaloStrided - 1;
      if (!tile_geometry<GP>(dtype, p, tg, halo, kPairStridedTH)) return hipErrorNotSupported;
    }
  } else if (!tile_geometry<GP>(dtype, p, tg, halo)) {
    if (GP != 1 || udil != 0) return hipErrorNotSupported;
    halo = kTileHaloSmall;
    if (!tile_geometry<GP>(dtype, p, tg, halo)) return hipErrorNotSupported;
  }
  if (p.RC) {  // fp32 only: 16-bit rows without the centre go to the lane kernel
    return dtype == DCN_F32 ? launch_tile_dt<DCN_F32, GP, true>(softmax, udil, halo, p, tg, s) : hipErrorNotSupported;
  }
  switch (dtype) {
    case DCN_F32: return launch_tile_dt<DCN_F32, GP, false>(softmax, udil, halo, p, tg, s);
    case DCN_F16: return launch_tile_dt<DCN_F16, GP, false>(softmax, udil, halo, p, tg, s);
    case DCN_BF16: return launch_tile_dt<DCN_BF16, GP, false>(softmax, udil, halo, p, tg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Returns hipErrorNotSupported (nothing launched) when the problem is not a
// 3x3 one (all nine points, or eight without the centre in fp32) or its
// window does not fit the LDS budget.  groups_per_item: 1 or
// 2 forces that variant; 0 takes two groups per item where they fit.
hipError_t launch_forward_tiled(int dtype, int softmax, const FwdParams &p, hipStream_t s, int groups_per_item) {
  if (p.KH != 3 || p.KW != 3) return hipErrorNotSupported;
  if (groups_per_item != 1) {
    const hipError_t e = launch_tile_gp<2>(dtype, softmax, p, s);
    if (e != hipErrorNotSupported || groups_per_item == 2) return e;
  }
  return launch_tile_gp<1>(dtype, softmax, p, s);
}

}  // namespace dcn
