// dcn_fwd_lane.hip -- LDS-tiled gfx950 forward kernel of the DCN core for
// 3x3 kernel points, one lane per pixel-group (wmrh.cn/news/61976, section 二
// steps 2-4 and section 三); also for the 8 points DCNv4's remove_center
// leaves (pnsm.cn/news/2029644.html section 3.3).
//
// The forward is a gather-reduce: per bilinear sample 64 fp32 FMAs (16
// channels x 4 corners) against a few dozen instructions of location and
// weight math.  With one lane per pixel-group that math is done exactly once
// per sample and needs no cross-lane broadcast; for 16-bit I/O each FMA takes
// its 16-bit operand directly (v_fma_mix), so no unpacking either.
//
// Block = one (image, output tile, block of GP groups) work item at a time,
// one lane per (pixel, group): 16x16 tiles, 16x8 or 24x8 with four groups
// (512 or 768 threads); blocks are persistent and each XCD walks one
// contiguous range of items.  The input window of an item (its regular 3x3
// footprint plus a halo of R pixels for the learned offsets, zero outside the
// map) is staged in LDS, the GP group slices of a window pixel side by side
// as they lie in memory: with four 16-bit groups a window pixel is one whole
// 128-byte line, which took the stage-2 launch from 1.74x to 1.00x of its
// algorithmic HBM bytes.  Each lane stages the same window pixels of every
// item (lane-constant slices of rows and columns), so the per-item address
// work is one add per slice.  The next item's window, offsets and logits are
// requested into registers while the current item computes.  A sample whose
// corners leave the window is served from global memory behind a wave
// ballot (the buffer range check supplying the zeros); the main path has no
// branches.
//
// LDS banking: a wave64 ds_read_b128 is served 16 lanes at a time from 64
// banks.  Lanes read the 16-byte chunks of a corner in a rotated order, so
// that pixels which share a bank row at unit offsets start on different
// chunks; the remaining conflicts are the random coincidences of the
// sampled pixels' bank quarters.
#include <algorithm>
#include <type_traits>

#include "dcn_device.hpp"

namespace dcn {

#ifndef DCN_LANE_HALO
#define DCN_LANE_HALO 6
#endif

constexpr int kLaneHalo = DCN_LANE_HALO;      // window halo for the offsets
// LDS bytes of a TW x TH tile's window for KS x KS points (and its zero
// block) at pixb bytes per staged window pixel.
template <int TW, int TH, int KS = 3>
constexpr int lane_lds_bytes(int pixb) {
  return ((TW + 2 * kLaneHalo + KS) * (TH + 2 * kLaneHalo + KS) + (TW + 2 * kLaneHalo + KS) + 2) * pixb;
}

// Bytes of one pixel-group (16 channels) in the I/O dtype.
template <int DT>
constexpr int lane_slice_bytes() { return kGroupChannels * Io<DT>::kBytes; }

namespace {

__device__ __forceinline__ void lds_read16(const unsigned char *src, uint32_t (&w)[4]) {
  const uint4 v = *reinterpret_cast<const uint4 *>(src);
  w[0] = v.x;
  w[1] = v.y;
  w[2] = v.z;
  w[3] = v.w;
}

// Words [0, N) of w from N consecutive words at byte offset `off` (4-byte
// aligned), in loads of at most 16 bytes.
template <int N, int M>
__device__ __forceinline__ void load_run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[M]) {
  static_assert(N <= M, "run length");
#pragma unroll
  for (int q = 0; q + 4 <= N; q += 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 4 * q), 0, 0);
    w[q] = v[0];
    w[q + 1] = v[1];
    w[q + 2] = v[2];
    w[q + 3] = v[3];
  }
  constexpr int B = N & ~3;
  if constexpr (N - B >= 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(off + 4 * B), 0, 0);
    w[B] = v[0];
    w[B + 1] = v[1];
  }
  if constexpr (N - B == 1 || N - B == 3)
    w[N - 1] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + 4 * (N - 1)), 0, 0);
}

// Offset and mask rows of one pixel-group for any number K of points, as
// raw words: fp32 2K offset words and K mask words; 16-bit K offset words
// (x, y per word) and the mask row's words from the 4-byte boundary at or
// below its start.  With K odd, 16-bit mask rows alternate between starting
// on a word and two bytes into one: a row that starts on a word takes its
// last value by a 2-byte load, so no load reaches past the row.
template <int DT, int K>
struct PointRows {
  static constexpr bool kF32 = DT == DCN_F32;
  static constexpr int kOff = kF32 ? 2 * K : K;
  static constexpr int kMask = kF32 ? K : (K % 2 == 0 ? K / 2 : (2 * K + 2) / 4);
  uint32_t o[kOff], m[kMask];
};

// The row words of a KS x KS problem: RowWords for 3x3 (nine or eight
// points), PointRows otherwise.
template <int DT, int K, int KS>
struct RowsOf {
  using type = PointRows<DT, K>;
};
template <int DT, int K>
struct RowsOf<DT, K, 3> {
  using type = RowWords<DT, K>;
};

template <int DT, int K, int KS>
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t roff, __amdgpu_buffer_rsrc_t rmask, uint32_t pg,
                                          typename RowsOf<DT, K, KS>::type &r) {
  if constexpr (KS == 3) {
    load_row_words<DT, K>(roff, rmask, pg, r);
  } else {
    using R = PointRows<DT, K>;
    load_run<R::kOff>(roff, pg * (uint32_t)(4 * R::kOff), r.o);
    if constexpr (R::kF32 || K % 2 == 0) {
      load_run<R::kMask>(rmask, pg * (uint32_t)(4 * R::kMask), r.m);
    } else {
      const uint32_t mb = pg * (uint32_t)(2 * K), a = mb & ~3u;
      const bool odd = (mb & 2u) != 0;
      load_run<R::kMask - 1>(rmask, a, r.m);
      const uint32_t last = a + 4u * (R::kMask - 1);
      const uint32_t wa = __builtin_amdgcn_raw_buffer_load_b32(rmask, odd ? (int)last : (int)kOutOfRange, 0, 0);
      const uint32_t wb = __builtin_amdgcn_raw_buffer_load_b16(rmask, odd ? (int)kOutOfRange : (int)last, 0, 0);
      r.m[R::kMask - 1] = wa | wb;
    }
  }
}

template <int DT, int K, int KS>
__device__ __forceinline__ void decode_mask(uint32_t pg, const typename RowsOf<DT, K, KS>::type &r,
                                            float (&msk)[K]) {
  if constexpr (KS == 3) {
    decode_mask_words<DT, K>(pg, r, msk);
  } else {
    using R = PointRows<DT, K>;
    if constexpr (R::kF32) {
#pragma unroll
      for (int q = 0; q < K; ++q) msk[q] = __uint_as_float(r.m[q]);
    } else {
      const uint32_t sh = (K % 2 != 0 && ((pg * (uint32_t)(2 * K)) & 2u)) ? 16u : 0u;  // row starts at a half word
      uint32_t w[R::kMask];
#pragma unroll
      for (int q = 0; q + 1 < R::kMask; ++q) w[q] = __builtin_amdgcn_alignbit(r.m[q + 1], r.m[q], sh);
      w[R::kMask - 1] = r.m[R::kMask - 1] >> sh;
#pragma unroll
      for (int q = 0; q < K; ++q) msk[q] = (q & 1) ? Io<DT>::hi(w[q / 2]) : Io<DT>::lo(w[q / 2]);
    }
  }
}

template <int DT, int K, int KS>
__device__ __forceinline__ void offset_xy(const typename RowsOf<DT, K, KS>::type &r, int k, float &x, float &y) {
  if constexpr (KS == 3) {
    offset_words_xy<DT, K>(r, k, x, y);
  } else if constexpr (DT == DCN_F32) {
    x = __uint_as_float(r.o[2 * k]);
    y = __uint_as_float(r.o[2 * k + 1]);
  } else {
    x = Io<DT>::lo(r.o[k]);
    y = Io<DT>::hi(r.o[k]);
  }
}

}  // namespace

// KS: the kernel's side (3 or 5).  RC: the centre point is removed (K =
// KS^2 - 1 points; point k sits at grid index k + (k >= KS^2 / 2)).  TW x
// TH: the output tile.  GP: groups per work item (1, 2
// or 4), one lane per (pixel, group), the GP lanes of a pixel adjacent.
// A staged window pixel holds the item's GP neighbouring group slices, which
// are contiguous in memory: with four 16-bit groups it is one whole 128-byte
// line, so the window costs a quarter of the line requests of one group per
// item, and the GP lanes of a pixel read one contiguous stretch of the
// offset and mask rows.
template <int DT, bool SOFTMAX, bool RC, int TW, int TH, int GP, int KS>
#ifndef DCN_LANE_WAVES
#define DCN_LANE_WAVES 2  // waves per SIMD the register budget must allow
#endif
__global__ void __launch_bounds__(TW * TH * GP, DCN_LANE_WAVES) dcn_fwd_lane_kernel(FwdParams p, TileGeom tg) {
  using io = Io<DT>;
  constexpr int THREADS = TW * TH * GP, R = kLaneHalo;
  constexpr int SPAN_W = TW + 2 * R + KS, SPAN_H = TH + 2 * R + KS;
  constexpr int GS = lane_slice_bytes<DT>();       // one pixel-group slice
  constexpr int PIXB = GS * GP;                    // one staged window pixel
  constexpr int CHUNK = 16;                        // bytes per ds_read_b128
  constexpr int NCH = GS / CHUNK;                  // chunks per slice: 4 (fp32) or 2
  constexpr int CPC = CHUNK / io::kBytes;          // channels per chunk: 4 or 8
  constexpr int ROW = SPAN_W * PIXB;               // LDS bytes per window row
  constexpr int SPAN = SPAN_W * SPAN_H;
  constexpr int LPP = PIXB / CHUNK;                // lanes staging one window pixel
  constexpr int WPIX = THREADS / LPP;              // window pixels per staging slice
  constexpr int LIM_X = SPAN_W - 2, LIM_Y = SPAN_H - 2;
  constexpr int ZERO = SPAN * PIXB;
  constexpr int K = KS * KS - (RC ? 1 : 0);
  constexpr int KC = KS * KS / 2;                  // the centre's grid index
  // 3x3 rows as RowWords (nine or eight points), others as PointRows.  The
  // next item's rows are requested before this item's compute, except for
  // 5x5 fp32 rows (75 words), which would not fit twice beside the window
  // prefetch: those are requested after it.
  using Rows = typename RowsOf<DT, K, KS>::type;
  constexpr bool EARLY_ROWS = KS == 3 || DT != DCN_F32;
  constexpr int BANK_PIX = 256 / PIXB;             // window pixels per 256-byte bank row
  static_assert(GP == 1 || GP == 2 || GP == 4, "one, two or four groups per item");
  static_assert(PIXB <= 128 && (PIXB & (PIXB - 1)) == 0 && THREADS % LPP == 0, "a window pixel is at most one line");

  // Window slices, the same window pixels for a lane in every item: main
  // slice u holds rows [u RPS, u RPS + RPS) of columns [0, CW), remainder
  // slices the rows below and the columns right of that block.  Per item a
  // slice costs one add; rows outside the map fall out of the image's buffer
  // range (negative or past its last byte) and read zero, and one column
  // check per slice rejects columns left or right of the map.
  constexpr int CW = SPAN_W > 32 ? 32 : SPAN_W;
  constexpr int RPS = WPIX / CW;
  constexpr int NM = SPAN_H / RPS;
  constexpr int REM_A = (SPAN_H - NM * RPS) * CW, REM_B = (SPAN_W - CW) * SPAN_H;
  constexpr int NR = (REM_A + REM_B + WPIX - 1) / WPIX;
  constexpr int NRA = NR > 0 ? NR : 1;
  constexpr int SLOTS = NM + NR;
  static_assert(RPS >= 1 && NM >= 1, "window slice mapping");

  extern __shared__ __align__(16) unsigned char tile[];

  const uint32_t lane = threadIdx.x;
  const uint32_t gsel = lane % GP, px = lane / GP;
  const int oy = (int)px / TW, ox = (int)px % TW;
  const uint32_t pix_bytes = (uint32_t)p.C * io::kBytes;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const uint32_t img_bytes = (uint32_t)p.H * row_bytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const __amdgpu_buffer_rsrc_t roff = make_rsrc(p.offset, p.off_bytes);
  const __amdgpu_buffer_rsrc_t rmask = make_rsrc(p.mask, p.mask_bytes);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(p.output, p.out_bytes);
  const float s = p.scale;
  const uint32_t gblocks = (uint32_t)p.G / GP;     // the launcher checks G % GP == 0

  // Zero block after the window (written once; ordered by the first barrier).
  for (int z = (int)lane * 16; z < ROW + 2 * PIXB; z += THREADS * 16)
    *reinterpret_cast<uint4 *>(tile + ZERO + z) = make_uint4(0, 0, 0, 0);

  // This lane's window slices: LPP lanes per window pixel, one 16-byte chunk each.
  const uint32_t slot = lane / LPP, sc = lane % LPP;
  const uint32_t m_col = slot % CW, m_row = slot / CW;
  const bool m_live = slot < (uint32_t)(RPS * CW);
  const uint32_t m_lane = m_row * row_bytes + m_col * pix_bytes + sc * CHUNK;
  const uint32_t m_lds = (m_row * SPAN_W + m_col) * PIXB + sc * CHUNK;
  uint32_t r_x[NRA], r_lane[NRA], r_lds[NRA];
  bool r_live[NRA];
#pragma unroll
  for (int rho = 0; rho < NR; ++rho) {
    const uint32_t rs = (uint32_t)rho * WPIX + slot;
    uint32_t y = 0, x = 0;
    if (rs < (uint32_t)REM_A) {
      y = NM * RPS + rs / CW;
      x = rs % CW;
    } else if constexpr (SPAN_W > CW) {
      y = (rs - REM_A) / (SPAN_W - CW);
      x = CW + (rs - REM_A) % (SPAN_W - CW);
    }
    r_live[rho] = rs < (uint32_t)(REM_A + REM_B);
    r_x[rho] = x;
    r_lane[rho] = y * row_bytes + x * pix_bytes + sc * CHUNK;
    r_lds[rho] = (y * SPAN_W + x) * PIXB + sc * CHUNK;
  }

  struct Item {
    uint32_t g0, g, n;
    int Y0, X0;
    bool live;
    uint32_t pg, rpg;  // rpg: the row the loads read (row 0 for a dead lane)
  };
  auto decode = [&](uint32_t it) {
    Item I;
    const uint32_t t = fast_div(it, tg.div_g);  // divides by the G / GP group blocks
    I.g0 = (it - t * gblocks) * GP;
    I.g = I.g0 + gsel;
    I.n = fast_div(t, tg.div_tiles);
    const uint32_t tile_id = t - I.n * (uint32_t)tg.tiles_per_img;
    const uint32_t tyi = fast_div(tile_id, tg.div_tiles_x);
    const uint32_t txi = tile_id - tyi * (uint32_t)tg.tiles_x;
    const int r0 = (int)tyi * TH, c0 = (int)txi * TW;
    I.Y0 = r0 - p.PH - R;  // window origin (stride and dilation 1)
    I.X0 = c0 - p.PW - R;
    const int ho = r0 + oy, wo = c0 + ox;
    I.live = ho < p.Ho && wo < p.Wo;
    I.pg = (((I.n * (uint32_t)p.Ho + ho) * (uint32_t)p.Wo + wo) * (uint32_t)p.G) + I.g;
    I.rpg = I.live ? I.pg : 0u;
    return I;
  };

  uint32_t win[SLOTS][4];
  auto issue_window = [&](const Item &I) {
    const __amdgpu_buffer_rsrc_t rimg =
        make_rsrc(static_cast<const unsigned char *>(p.input) + (size_t)I.n * img_bytes, img_bytes);
    const uint32_t base = (uint32_t)I.Y0 * row_bytes + (uint32_t)I.X0 * pix_bytes + I.g0 * GS;  // mod 2^32
    const uint32_t m_off = m_live && (uint32_t)(I.X0 + (int)m_col) < (uint32_t)p.W ? base + m_lane : kOutOfRange;
#pragma unroll
    for (int u = 0; u < NM; ++u) buffer_load_words<4>(rimg, m_off + (uint32_t)(u * RPS) * row_bytes, win[u]);
#pragma unroll
    for (int rho = 0; rho < NR; ++rho) {
      const uint32_t r_off = r_live[rho] && (uint32_t)(I.X0 + (int)r_x[rho]) < (uint32_t)p.W
                                 ? base + r_lane[rho] : kOutOfRange;
      buffer_load_words<4>(rimg, r_off, win[NM + rho]);
    }
  };
  auto store_window = [&]() {
    if (m_live) {
#pragma unroll
      for (int u = 0; u < NM; ++u)
        *reinterpret_cast<uint4 *>(tile + m_lds + u * RPS * ROW) = make_uint4(win[u][0], win[u][1], win[u][2], win[u][3]);
    }
#pragma unroll
    for (int rho = 0; rho < NR; ++rho)
      if (r_live[rho])
        *reinterpret_cast<uint4 *>(tile + r_lds[rho]) =
            make_uint4(win[NM + rho][0], win[NM + rho][1], win[NM + rho][2], win[NM + rho][3]);
  };

  // Offsets and logits of the next item, as the raw words the buffer loads
  // return: decoded after the next window is in LDS, so the loads overlap a
  // whole item of compute.  Issued on every path (a dead lane reads row 0),
  // so the compiler's wait counting stays exact.
  Rows rw;

  // Per-lane chunk order (bank spreading): the pixels that share a bank row
  // at unit offsets start on different chunks.
  int rot[NCH];
#pragma unroll
  for (int t = 0; t < NCH; ++t) rot[t] = ((t + (int)px / BANK_PIX) % NCH) * CHUNK;

  const XcdWalk walk = xcd_walk(blockIdx.x, gridDim.x, tg.items);
  const uint32_t end = walk.end;
  uint32_t item = walk.first;
  Item cur = decode(item < end ? item : 0);
  if (item < end) {
    issue_window(cur);
    load_rows<DT, K, KS>(roff, rmask, cur.rpg, rw);
  }

  while (item < end) {
    __syncthreads();  // every wave is done with the previous window
    store_window();
    __syncthreads();  // the window is in LDS

    // This item's rows (the offsets are decoded point by point).
    const Rows cw = rw;

    // The next item's window and rows land in registers during this item's
    // compute.  (Issued on the last item too, re-reading its own data, so
    // that no branch changes the count of outstanding loads.)
    const uint32_t next = item + walk.stride;
    const bool more = next < end;  // block-uniform
    const Item nx = decode(more ? next : item);
    issue_window(nx);
    if constexpr (EARLY_ROWS) load_rows<DT, K, KS>(roff, rmask, nx.rpg, rw);

    // modulation scalars
    float msk[K], m[K];
    decode_mask<DT, K, KS>(cur.rpg, cw, msk);
    if constexpr (SOFTMAX) {
      float mx = msk[0];
#pragma unroll
      for (int k = 1; k < K; ++k) mx = fmaxf(mx, msk[k]);
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        m[k] = __expf(msk[k] - mx);
        sum += m[k];
      }
      const float inv = __builtin_amdgcn_rcpf(sum);
#pragma unroll
      for (int k = 0; k < K; ++k) m[k] *= inv;
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) m[k] = msk[k];
    }

    float acc[NCH][CPC];
#pragma unroll
    for (int t = 0; t < NCH; ++t)
#pragma unroll
      for (int c = 0; c < CPC; ++c) acc[t][c] = 0.f;

    const uint32_t img = cur.n * img_bytes;
    const uint32_t chan = cur.g * GS;
    const unsigned char *slice = tile + gsel * GS;  // this lane's group in a window pixel

#pragma unroll
    for (int k = 0; k < K; ++k) {
      // Wave priority falls as the wave moves through the points, so the
      // waves furthest behind issue first and the block reaches its next
      // barrier with less spread.
      if (k == 0) __builtin_amdgcn_s_setprio(3);
      if (k == (KS == 3 ? 3 : K / 3)) __builtin_amdgcn_s_setprio(2);
      if (k == (KS == 3 ? 6 : 2 * K / 3)) __builtin_amdgcn_s_setprio(1);
      const int q = RC ? k + (k >= KC) : k;  // grid index
      const int i = q / KS, j = q % KS;
      float ox_k, oy_k;
      offset_xy<DT, K, KS>(cw, k, ox_k, oy_k);
      const float dx = s * ox_k, dy = s * oy_k;
      const bool nan_loc = (dx != dx) | (dy != dy);
      const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
      const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
      const float fx = floorf(cx), fy = floorf(cy);
      const float lx = cx - fx, ly = cy - fy;
      // window coordinates: regular position oy + i + R (stride/dilation 1)
      const int ty = oy + i + R + (int)fy, tx = ox + j + R + (int)fx;
      const float mk = nan_loc ? __builtin_nanf("") : m[k];
      const float wy0 = (1.f - ly) * mk, wy1 = ly * mk;
      const float w00 = wy0 * (1.f - lx), w01 = wy0 * lx;
      const float w10 = wy1 * (1.f - lx), w11 = wy1 * lx;
      const bool inside = !nan_loc && (uint32_t)ty <= (uint32_t)LIM_Y && (uint32_t)tx <= (uint32_t)LIM_X;
      // (24-bit multiply: an inside ty is below the span)
      const uint32_t A = inside ? (uint32_t)__umul24((uint32_t)ty, (uint32_t)ROW) + (uint32_t)tx * PIXB : (uint32_t)ZERO;
      const unsigned char *src = slice + A;
#pragma unroll
      for (int t = 0; t < NCH; ++t) {
        const unsigned char *q = src + rot[t];
        uint32_t v00[4], v01[4], v10[4], v11[4];
        lds_read16(q, v00);
        lds_read16(q + PIXB, v01);
        lds_read16(q + ROW, v10);
        lds_read16(q + ROW + PIXB, v11);
        float f00[CPC], f01[CPC], f10[CPC], f11[CPC];
        unpack<DT, 4>(v00, f00);
        unpack<DT, 4>(v01, f01);
        unpack<DT, 4>(v10, f10);
        unpack<DT, 4>(v11, f11);
#pragma unroll
        for (int c = 0; c < CPC; ++c) {
          acc[t][c] = fmaf(w00, f00[c], acc[t][c]);
          acc[t][c] = fmaf(w01, f01[c], acc[t][c]);
          acc[t][c] = fmaf(w10, f10[c], acc[t][c]);
          acc[t][c] = fmaf(w11, f11[c], acc[t][c]);
        }
        pin_values(acc[t]);  // the chunk's FMAs happen here, not at the end
      }
      // Corners outside the window but touching the map: global gathers
      // (rare; the wave skips this when no lane needs it).
      const bool fb = !inside && !nan_loc;
      if (__builtin_amdgcn_ballot_w64(fb) != 0) {
        if (fb) {
          const int y0 = cur.Y0 + ty, x0 = cur.X0 + tx;
          const bool vy0 = (uint32_t)y0 < (uint32_t)p.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)p.H;
          const bool vx0 = (uint32_t)x0 < (uint32_t)p.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)p.W;
          const uint32_t a00 = img + (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_bytes + chan;
#pragma unroll
          for (int t = 0; t < NCH; ++t) {
            uint32_t v00[4], v01[4], v10[4], v11[4];
            const uint32_t ct = (uint32_t)rot[t];
            buffer_load_words<4>(rin, (vy0 && vx0) ? a00 + ct : kOutOfRange, v00);
            buffer_load_words<4>(rin, (vy0 && vx1) ? a00 + pix_bytes + ct : kOutOfRange, v01);
            buffer_load_words<4>(rin, (vy1 && vx0) ? a00 + row_bytes + ct : kOutOfRange, v10);
            buffer_load_words<4>(rin, (vy1 && vx1) ? a00 + row_bytes + pix_bytes + ct : kOutOfRange, v11);
            float f00[CPC], f01[CPC], f10[CPC], f11[CPC];
            unpack<DT, 4>(v00, f00);
            unpack<DT, 4>(v01, f01);
            unpack<DT, 4>(v10, f10);
            unpack<DT, 4>(v11, f11);
#pragma unroll
            for (int c = 0; c < CPC; ++c) {
              acc[t][c] = fmaf(w00, f00[c], acc[t][c]);
              acc[t][c] = fmaf(w01, f01[c], acc[t][c]);
              acc[t][c] = fmaf(w10, f10[c], acc[t][c]);
              acc[t][c] = fmaf(w11, f11[c], acc[t][c]);
            }
          }
        }
      }
    }

    // acc[t] holds the chunk at byte offset rot[t] of the 16-channel slice;
    // a dead lane's store carries an out-of-range offset and is dropped.
    const uint32_t obase = cur.live ? cur.pg * (uint32_t)GS : kOutOfRange;
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
      uint32_t w[4];
      pack_words<DT, CPC>(acc[t], w);
      buffer_store_words<4>(rout, obase + (uint32_t)rot[t], w);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (!EARLY_ROWS) load_rows<DT, K, KS>(roff, rmask, nx.rpg, rw);

    item = next;
    cur = nx;
  }
}

namespace {

#ifndef DCN_LANE_GP_MAX
#define DCN_LANE_GP_MAX 4
#endif
#ifndef DCN_LANE_TH4
#define DCN_LANE_TH4 8  // height of the 16-wide tiles with four groups per item
#endif

template <int DT, bool SM, bool RC, int TW, int TH, int GP, int KS>
hipError_t launch_lane(const FwdParams &p, const TileGeom &tg, hipStream_t s) {
  auto kern = dcn_fwd_lane_kernel<DT, SM, RC, TW, TH, GP, KS>;
  constexpr int THREADS = TW * TH * GP;
  const size_t lds = lane_lds_bytes<TW, TH, KS>(lane_slice_bytes<DT>() * GP);
  // Set on every launch: the limit is per device and setting it is idempotent.
  const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // Persistent blocks: as many per CU as are resident together (registers
  // and LDS permitting), so no block waits for another to finish.
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern),
                                                   THREADS, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorNotSupported;
  const uint32_t blocks = std::min<uint32_t>(tg.items, (uint32_t)per_cu * (uint32_t)cus);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(THREADS), lds, s, p, tg);
  return hipGetLastError();
}

// Tile shape of each kind of work item: 16 x 16, or 16 x 8 with four
// groups (a 1024-thread block would have half the registers per lane), or
// 24 x 8 (16-bit, 3x3 points).
struct LaneShape {
  int tw, th;
};

LaneShape lane_shape(bool wide, int gp) {
  if (wide) return LaneShape{24, 8};
  return gp == 4 ? LaneShape{16, DCN_LANE_TH4} : LaneShape{16, 16};
}

template <int DT, bool SM, bool RC, int KS>
hipError_t launch_lane_shape(bool wide, int gp, const FwdParams &p, const TileGeom &tg, hipStream_t s) {
  if constexpr (DT == DCN_F32) {  // one group per item, 16x16 tiles (the 24x8 window would need 19 slots per lane)
    if (wide || gp != 1) return hipErrorNotSupported;
    return launch_lane<DT, SM, RC, 16, 16, 1, KS>(p, tg, s);
  } else if constexpr (KS == 5) {  // 16-wide tiles only
    if (wide) return hipErrorNotSupported;
    if (gp == 4) return launch_lane<DT, SM, RC, 16, DCN_LANE_TH4, 4, KS>(p, tg, s);
    return launch_lane<DT, SM, RC, 16, 16, 1, KS>(p, tg, s);
  } else {
    if (gp == 4)
      return wide ? launch_lane<DT, SM, RC, 24, 8, 4, KS>(p, tg, s) : launch_lane<DT, SM, RC, 16, DCN_LANE_TH4, 4, KS>(p, tg, s);
    if (gp == 2)
      return wide ? launch_lane<DT, SM, RC, 24, 8, 2, KS>(p, tg, s) : launch_lane<DT, SM, RC, 16, 16, 2, KS>(p, tg, s);
    return wide ? launch_lane<DT, SM, RC, 24, 8, 1, KS>(p, tg, s) : launch_lane<DT, SM, RC, 16, 16, 1, KS>(p, tg, s);
  }
}

template <int DT, int KS>
hipError_t launch_lane_dt(bool wide, int gp, int softmax, const FwdParams &p, const TileGeom &tg, hipStream_t s) {
  if (p.RC)
    return softmax ? launch_lane_shape<DT, true, true, KS>(wide, gp, p, tg, s)
                   : launch_lane_shape<DT, false, true, KS>(wide, gp, p, tg, s);
  return softmax ? launch_lane_shape<DT, true, false, KS>(wide, gp, p, tg, s)
                 : launch_lane_shape<DT, false, false, KS>(wide, gp, p, tg, s);
}

// Share of the tiles' lanes that hold an output pixel.
double lane_use(const FwdParams &p, int tw, int th) {
  const double tiled = (double)((p.Ho + th - 1) / th) * th * (double)((p.Wo + tw - 1) / tw) * tw;
  return (double)p.Ho * p.Wo / tiled;
}

}  // namespace

// 3x3 or 5x5 points, stride 1, dilation 1; hipErrorNotSupported otherwise.
// 16-bit I/O takes four groups per work item where the group count allows
// (3x3: two, else one; 5x5: see below), fp32 one.
hipError_t launch_forward_lane(int dtype, int softmax, const FwdParams &p, hipStream_t s) {
  if (p.KH != p.KW || (p.KH != 3 && p.KH != 5) || p.SH != 1 || p.SW != 1 || p.DH != 1 || p.DW != 1)
    return hipErrorNotSupported;
  if (dtype != DCN_F32 && dtype != DCN_F16 && dtype != DCN_BF16) return hipErrorInvalidValue;
  const int ks = p.KH;
  int gp = 1;
  if (dtype != DCN_F32) {
    if (p.G % 4 == 0 && DCN_LANE_GP_MAX >= 4) gp = 4;
    else if (p.G % 2 == 0 && DCN_LANE_GP_MAX >= 2) gp = 2;
  }
  // 5x5 (16-bit): one group per item on 16x16 tiles (a third more blocks
  // per CU than four groups on 16x8 tiles: 0.46 against 0.54 ms at stage-2
  // size), unless those tiles leave clearly more lanes idle (the 24x24
  // stage: 56 % full against 75 %; 0.53 against 0.43 ms)
  if (ks == 5 && gp != 1)
    gp = (p.G % 4 == 0 && DCN_LANE_GP_MAX >= 4 && lane_use(p, 16, DCN_LANE_TH4) > lane_use(p, 16, 16) + 0.1) ? 4 : 1;
  const LaneShape sq = lane_shape(false, gp), sw = lane_shape(true, gp);
  // 24x8 tiles (16-bit, 3x3) where they leave clearly fewer lanes idle; with
  // four groups also where they leave as few (768 threads, twelve waves,
  // against 512 on 16x8 tiles, and fewer halo pixels per output pixel: 4.7
  // against 5.6)
  const double use_w = lane_use(p, sw.tw, sw.th), use_q = lane_use(p, sq.tw, sq.th);
  const bool wide = dtype != DCN_F32 && ks == 3 && (use_w > use_q + 0.1 || (gp == 4 && use_w >= use_q));
  const LaneShape sh = wide ? sw : sq;
  TileGeom tg{};
  tg.span_w = sh.tw + 2 * kLaneHalo + ks;
  tg.span_h = sh.th + 2 * kLaneHalo + ks;
  // The window rows above and below the map are rejected by the buffer range
  // of their image, which needs the byte offset of every window row relative
  // to the image to fit int32.
  const int64_t row_bytes = (int64_t)p.W * p.C * (dtype == DCN_F32 ? 4 : 2);
  if (((int64_t)p.H + p.PH + tg.span_h + 1) * row_bytes >= (int64_t(1) << 31)) return hipErrorNotSupported;
  const int tiles_y = (p.Ho + sh.th - 1) / sh.th;
  tg.tiles_x = (p.Wo + sh.tw - 1) / sh.tw;
  tg.tiles_per_img = tiles_y * tg.tiles_x;
  const int64_t imgs = p.pg_total / ((int64_t)p.Ho * p.Wo * p.G);
  const int64_t items = imgs * tg.tiles_per_img * (p.G / gp);
  if (items <= 0 || items >= (int64_t(1) << 31)) return hipErrorNotSupported;
  tg.items = (uint32_t)items;
  tg.div_g = make_fast_div((uint32_t)(p.G / gp));  // group blocks per tile
  tg.div_tiles = make_fast_div((uint32_t)tg.tiles_per_img);
  tg.div_tiles_x = make_fast_div((uint32_t)tg.tiles_x);
  tg.div_span_w = make_fast_div((uint32_t)tg.span_w);
  if (ks == 5) {
    switch (dtype) {
      case DCN_F32: return launch_lane_dt<DCN_F32, 5>(wide, gp, softmax, p, tg, s);
      case DCN_F16: return launch_lane_dt<DCN_F16, 5>(wide, gp, softmax, p, tg, s);
      default: return launch_lane_dt<DCN_BF16, 5>(wide, gp, softmax, p, tg, s);
    }
  }
  switch (dtype) {
    case DCN_F32: return launch_lane_dt<DCN_F32, 3>(wide, gp, softmax, p, tg, s);
    case DCN_F16: return launch_lane_dt<DCN_F16, 3>(wide, gp, softmax, p, tg, s);
    default: return launch_lane_dt<DCN_BF16, 3>(wide, gp, softmax, p, tg, s);
  }
}

}  // namespace dcn
