// dcn_fwd_lane.hip -- LDS-tiled gfx950 forward kernel of the DCN core for
// 3x3 kernel points, one lane per pixel-group (wmrh.cn/news/61976, section 二
// steps 2-4 and section 三); also for the 8 points DCNv4's remove_center
// leaves (pnsm.cn/news/2029644.html section 3.3).
//
// The forward is a gather-reduce: per bilinear sample 64 fp32 FMAs (16
// channels x 4 corners) against a few dozen instructions of location and
// weight math.  With one lane per pixel-group that math is done exactly once
// per sample and needs no cross-lane broadcast, so the instruction stream is
// dominated by the FMAs themselves (vector fp32 issue is the binding limit on
// this chip once the corners come from LDS).
//
// Block = 256 threads = one (image, 16x16 output tile, group) work item at a
// time; blocks are persistent and each XCD walks one contiguous range of items.
// The input window of an item (its regular 3x3 footprint plus a halo of R
// pixels for the learned offsets, zero outside the map) is staged in LDS; the
// next item's window, offsets and logits are requested into registers while
// the current item computes.  A sample whose corners leave the window is
// served from global memory behind a wave ballot (the buffer range check
// supplying the zeros); the main path has no branches.
//
// LDS banking: a wave64 ds_read_b128 is served 16 lanes at a time from 64
// banks.  Lane l reads the 16-byte chunks of a corner in the rotated order
// (t + l) mod 4, so the four lanes that share a chunk position come from four
// different pixels; the remaining conflicts are the random coincidences of
// those pixels' bank quarters.
#include <algorithm>

#include "dcn_device.hpp"

namespace dcn {

#ifndef DCN_LANE_HALO
#define DCN_LANE_HALO 6
#endif

constexpr int kLaneHalo = DCN_LANE_HALO;      // window halo for the offsets
// Output tiles: 16x16 (256 lanes), or 24x8 (192 lanes, three waves) for
// maps 24 pixels wide, which 16x16 tiles would leave 44 % empty.
template <int TW, int TH>
constexpr int lane_lds_bytes(int pixb) {
  return ((TW + 2 * kLaneHalo + 3) * (TH + 2 * kLaneHalo + 3) + (TW + 2 * kLaneHalo + 3) + 2) * pixb;
}

template <int DT>
constexpr int lane_pixel_stride() { return DT == DCN_F32 ? 64 : 32; }

namespace {

__device__ __forceinline__ void lds_read16(const unsigned char *src, uint32_t (&w)[4]) {
  const uint4 v = *reinterpret_cast<const uint4 *>(src);
  w[0] = v.x;
  w[1] = v.y;
  w[2] = v.z;
  w[3] = v.w;
}

}  // namespace

// RC: the centre point is removed (8 points; point k sits at grid index
// k + (k >= 4)).  TW x TH: the output tile, one lane per pixel.
template <int DT, bool SOFTMAX, bool RC, int TW, int TH>
#ifndef DCN_LANE_WAVES
#define DCN_LANE_WAVES 2  // waves per SIMD the register budget must allow
#endif
__global__ void __launch_bounds__(TW * TH, DCN_LANE_WAVES) dcn_fwd_lane_kernel(FwdParams p, TileGeom tg) {
  using io = Io<DT>;
  constexpr int THREADS = TW * TH, R = kLaneHalo;
  constexpr int SPAN_W = TW + 2 * R + 3, SPAN_H = TH + 2 * R + 3;
  constexpr int CG = kGroupChannels;
  constexpr int PIXB = lane_pixel_stride<DT>();   // one pixel's 16-channel slice
  constexpr int CHUNK = 16;                        // bytes per ds_read_b128
  constexpr int NCH = PIXB / CHUNK;                // chunks per slice: 4 (fp32) or 2
  constexpr int CPC = CHUNK / io::kBytes;          // channels per chunk: 4 or 8
  constexpr int ROW = SPAN_W * PIXB;               // LDS bytes per window row
  constexpr int SPAN = SPAN_W * SPAN_H;
  constexpr int QUADS = THREADS / NCH;             // lanes groups staging one pixel each
  constexpr int SLOTS = (SPAN + QUADS - 1) / QUADS;
  constexpr int LIM_X = SPAN_W - 2, LIM_Y = SPAN_H - 2;
  constexpr int ZERO = SPAN * PIXB;
  constexpr int K = RC ? 8 : 9;

  extern __shared__ __align__(16) unsigned char tile[];

  const uint32_t lane = threadIdx.x;
  const int oy = (int)lane / TW, ox = (int)lane % TW;
  const uint32_t pix_bytes = (uint32_t)p.C * io::kBytes;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(p.output, p.pg_total * (uint32_t)(CG * io::kBytes));
  const float s = p.scale;

  // Zero block after the window (written once; ordered by the first barrier).
  for (int z = (int)lane * 16; z < ROW + 2 * PIXB; z += THREADS * 16)
    *reinterpret_cast<uint4 *>(tile + ZERO + z) = make_uint4(0, 0, 0, 0);

  // Staging: NCH lanes per pixel, SLOTS pixels per lane group.
  const uint32_t sq = lane / NCH, sc = lane % NCH;

  struct Item {
    uint32_t g, n;
    int Y0, X0, ho, wo;
    bool live;
    uint32_t pg;
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
    I.Y0 = r0 - p.PH - R;  // window origin (stride and dilation 1)
    I.X0 = c0 - p.PW - R;
    I.ho = r0 + oy;
    I.wo = c0 + ox;
    I.live = I.ho < p.Ho && I.wo < p.Wo;
    I.pg = (((I.n * (uint32_t)p.Ho + I.ho) * (uint32_t)p.Wo + I.wo) * (uint32_t)p.G) + I.g;
    return I;
  };

  uint32_t win[SLOTS][4];
  auto issue_window = [&](const Item &I) {
    const uint32_t base = I.n * (uint32_t)p.H * row_bytes + (I.g * CG) * io::kBytes + sc * CHUNK;
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const int idx = (int)sq + u * QUADS;
      const int sy = idx / SPAN_W, sx = idx - sy * SPAN_W;  // constant divisor
      const int gy = I.Y0 + sy, gx = I.X0 + sx;
      const bool ok = idx < SPAN && (uint32_t)gy < (uint32_t)p.H && (uint32_t)gx < (uint32_t)p.W;
      const uint32_t offb = ok ? base + (uint32_t)gy * row_bytes + (uint32_t)gx * pix_bytes : kOutOfRange;
      buffer_load_words<4>(rin, offb, win[u]);
    }
  };
  auto store_window = [&]() {
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const int idx = (int)sq + u * QUADS;
      if (idx < SPAN)
        *reinterpret_cast<uint4 *>(tile + idx * PIXB + sc * CHUNK) =
            make_uint4(win[u][0], win[u][1], win[u][2], win[u][3]);
    }
  };

  float off[2 * K], msk[K];
  // Unconditional (a dead lane reads pixel-group 0 and ignores it): every
  // memory instruction of the item loop is issued on every path, so the
  // compiler's wait counting stays exact and the window prefetch is only
  // waited for where the LDS store needs it.
  auto issue_pgdata = [&](const Item &I) {
    const uint32_t pg = I.live ? I.pg : 0u;
    load_offsets<DT, K>(p.offset, pg, off);
    load_mask<DT, K>(p.mask, pg, msk);
  };

  // Per-lane chunk rotation (bank spreading) and its byte offsets.
  int rot[NCH];
#pragma unroll
  for (int t = 0; t < NCH; ++t) rot[t] = ((t + (int)lane) % NCH) * CHUNK;

  const XcdWalk walk = xcd_walk(blockIdx.x, gridDim.x, tg.items);
  const uint32_t end = walk.end;
  uint32_t item = walk.first;
  Item cur = decode(item < end ? item : 0);
  if (item < end) {
    issue_window(cur);
    issue_pgdata(cur);
  }

  while (item < end) {
    __syncthreads();  // every wave is done with the previous window
    store_window();
    __syncthreads();  // the window is in LDS

    // The next item's window lands in registers during this item's compute;
    // its offsets and logits are requested once this item's are consumed.
    // (Issued on the last item too, re-reading its own data, so that no
    // branch changes the count of outstanding loads.)
    const uint32_t next = item + walk.stride;
    const bool more = next < end;  // block-uniform
    const Item nx = decode(more ? next : item);
    issue_window(nx);

    {
      // modulation scalars
      float m[K];
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

      const uint32_t img = cur.n * (uint32_t)p.H * row_bytes;
      const uint32_t chan = (cur.g * CG) * io::kBytes;

#pragma unroll
      for (int k = 0; k < K; ++k) {
        // Wave priority falls as the wave moves through the points, so the
        // waves furthest behind issue first and the block reaches its next
        // barrier with less spread.
        if (k == 0) __builtin_amdgcn_s_setprio(3);
        if (k == 3) __builtin_amdgcn_s_setprio(2);
        if (k == 6) __builtin_amdgcn_s_setprio(1);
        const int q = RC ? k + (k >= 4) : k;  // grid index
        const int i = q / 3, j = q % 3;
        const float dx = s * off[2 * k], dy = s * off[2 * k + 1];
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
        const int A = inside ? ty * ROW + tx * PIXB : ZERO;
        const unsigned char *src = tile + A;
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
      const uint32_t obase = cur.live ? cur.pg * (uint32_t)(CG * io::kBytes) : kOutOfRange;
#pragma unroll
      for (int t = 0; t < NCH; ++t) {
        uint32_t w[4];
        pack_words<DT, CPC>(acc[t], w);
        buffer_store_words<4>(rout, obase + (uint32_t)rot[t], w);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    issue_pgdata(nx);

    item = next;
    cur = nx;
  }
}

namespace {

template <int DT, bool SM, bool RC, int TW, int TH>
hipError_t launch_lane(const FwdParams &p, const TileGeom &tg, hipStream_t s) {
  auto kern = dcn_fwd_lane_kernel<DT, SM, RC, TW, TH>;
  constexpr int THREADS = TW * TH;
  const size_t lds = lane_lds_bytes<TW, TH>(lane_pixel_stride<DT>());
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

template <bool RC, int TW, int TH>
hipError_t launch_lane_dt(int dtype, int softmax, const FwdParams &p, const TileGeom &tg, hipStream_t s) {
  switch (dtype) {
    case DCN_F32:
      if constexpr (TW == 16) {  // the 24x8 tile is 16-bit only (fp32 would need 19 window slots per lane)
        return softmax ? launch_lane<DCN_F32, true, RC, TW, TH>(p, tg, s) : launch_lane<DCN_F32, false, RC, TW, TH>(p, tg, s);
      } else {
        return hipErrorNotSupported;
      }
    case DCN_F16:
      return softmax ? launch_lane<DCN_F16, true, RC, TW, TH>(p, tg, s) : launch_lane<DCN_F16, false, RC, TW, TH>(p, tg, s);
    case DCN_BF16:
      return softmax ? launch_lane<DCN_BF16, true, RC, TW, TH>(p, tg, s) : launch_lane<DCN_BF16, false, RC, TW, TH>(p, tg, s);
    default: return hipErrorInvalidValue;
  }
}

// Share of the tiles' lanes that hold an output pixel.
double lane_use(const FwdParams &p, int tw, int th) {
  const double tiled = (double)((p.Ho + th - 1) / th) * th * (double)((p.Wo + tw - 1) / tw) * tw;
  return (double)p.Ho * p.Wo / tiled;
}

}  // namespace

// Stride 1, dilation 1, 3x3 points only; hipErrorNotSupported otherwise.
hipError_t launch_forward_lane(int dtype, int softmax, const FwdParams &p, hipStream_t s) {
  if (p.KH != 3 || p.KW != 3 || p.SH != 1 || p.SW != 1 || p.DH != 1 || p.DW != 1)
    return hipErrorNotSupported;
  // 24x8 tiles (16-bit) where they leave clearly fewer lanes idle than 16x16
  const bool wide = dtype != DCN_F32 && lane_use(p, 24, 8) > lane_use(p, 16, 16) + 0.1;
  const int tw = wide ? 24 : 16, th = wide ? 8 : 16;
  TileGeom tg{};
  tg.span_w = tw + 2 * kLaneHalo + 3;
  tg.span_h = th + 2 * kLaneHalo + 3;
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
  if (wide)
    return p.RC ? launch_lane_dt<true, 24, 8>(dtype, softmax, p, tg, s) : launch_lane_dt<false, 24, 8>(dtype, softmax, p, tg, s);
  return p.RC ? launch_lane_dt<true, 16, 16>(dtype, softmax, p, tg, s) : launch_lane_dt<false, 16, 16>(dtype, softmax, p, tg, s);
}

}  // namespace dcn
