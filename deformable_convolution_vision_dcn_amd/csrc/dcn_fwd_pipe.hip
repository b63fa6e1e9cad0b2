// dcn_fwd_pipe.hip -- pipelined LDS-tiled gfx950 forward kernel of the DCN
// core for 3x3 kernel points at stride 1 and dilation 1 (wmrh.cn/news/61976,
// section 二 steps 2-4 and section 三).
//
// One lane per pixel-group: the location and weight arithmetic of a sample
// runs once per work item and feeds every channel, with no cross-lane
// traffic.  A block of 256 lanes owns one (image, 16x16 output tile, group)
// work item at a time and walks its XCD's range of items; two blocks per CU.
//
// The window (the tile's 3x3 footprint plus a halo of R pixels, zero outside
// the map) goes through LDS 32 bytes per pixel at a time: the whole 16-channel
// slice for 16-bit I/O, and two passes of 8 channels for fp32.  That keeps a
// window buffer at 32 KB, so each block double-buffers: while one pass is
// computed from one buffer, the next pass's window streams into the other
// with direct global->LDS loads (buffer_load_dwordx4 ... lds: lane l's 16
// bytes land at M0 + 16 l) and, at the last pass of an item, the next item's
// offsets and logits stream into registers.  The nine points' locations and
// weights are computed once per item and kept in registers for both passes.
// One barrier per pass.
//
// The DMA is issued from inline asm (M0 set in the same statement, no register
// outputs): the compiler cannot prove that reads of the other buffer do not
// alias a DMA it knows of and would wait for the DMA before each of them.
// Here it is waited for explicitly, once per pass, before the barrier; the
// previous pass's output is stored after that barrier, so the wait never
// covers fresh stores.
//
// Inside a pass the gathers of point k+1 are issued before point k's FMAs.
// Samples that leave the window read a zero block on the main path and are
// fixed up from global memory after the pass's window work (the buffer range
// check reads 0 for corners outside the map).  A lane reads the two 16-byte
// chunks of a corner in the order (t + lane) mod 2 to spread LDS banks.
#include <algorithm>

#include "dcn_device.hpp"

namespace dcn {

constexpr int kPipeTile = 16;
constexpr int kPipeHalo = 6;
constexpr int kPipeSpan = kPipeTile + 2 * kPipeHalo + 3;  // window edge, pixels
constexpr int kPipeThreads = kPipeTile * kPipeTile;
constexpr int kPipeSlice = 32;                            // LDS bytes per window pixel per pass
constexpr int kPipeWin = kPipeSpan * kPipeSpan * kPipeSlice;
// One buffer: the window, then a zero block of a row plus two pixels (what a
// sample outside the window reads), rounded to whole 1 KB DMA blocks.
constexpr int kPipeBuf = (kPipeWin + kPipeSpan * kPipeSlice + 2 * kPipeSlice + 1023) / 1024 * 1024;
constexpr int kPipeDma = (kPipeWin + 1023) / 1024;        // 1 KB DMA blocks per window
constexpr int kPipeBlocksPerCu = 2;

namespace {

__device__ __forceinline__ void lds_read16(const unsigned char *src, uint32_t (&w)[4]) {
  const uint4 v = *reinterpret_cast<const uint4 *>(src);
  w[0] = v.x;
  w[1] = v.y;
  w[2] = v.z;
  w[3] = v.w;
}

// 64 lanes x 16 bytes from the buffer resource into LDS at lds_base (wave
// uniform, bytes) + 16 * lane.  An out-of-range voff writes zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(r)
               : "memory");
}

}  // namespace

template <int DT, bool SOFTMAX>
__global__ void __launch_bounds__(kPipeThreads, kPipeBlocksPerCu)
    dcn_fwd_pipe_kernel(FwdParams p, TileGeom tg) {
  using io = Io<DT>;
  constexpr int TS = kPipeTile, R = kPipeHalo, SPAN_W = kPipeSpan;
  constexpr int CG = kGroupChannels;
  constexpr int PIXB = kPipeSlice;
  constexpr int CHUNK = 16;
  constexpr int NCH = PIXB / CHUNK;          // chunks per pass slice: 2
  constexpr int CPC = CHUNK / io::kBytes;    // channels per chunk: 4 or 8
  constexpr int CPP = NCH * CPC;             // channels per pass: 8 or 16
  constexpr int NH = CG / CPP;               // passes per item: 2 or 1
  constexpr int ROW = SPAN_W * PIXB;
  constexpr int SPAN = SPAN_W * SPAN_W;
  constexpr int LIM = SPAN_W - 2;
  constexpr int ZERO = kPipeWin;
  constexpr int BUF = kPipeBuf;
  constexpr int NDMA = kPipeDma;
  constexpr int WAVES = kPipeThreads / 64;
  constexpr int SLOTS = (NDMA + WAVES - 1) / WAVES;  // DMA blocks per wave
  constexpr int K = 9;
  static_assert(NDMA * 1024 <= BUF, "the last DMA block stays inside the buffer");
  static_assert(SPAN_W < 256, "window coordinates are packed in bytes");

  extern __shared__ __align__(16) unsigned char lds[];

  const uint32_t lane = threadIdx.x;
  const uint32_t wl = lane & 63, wave = lane >> 6;
  const int oy = (int)lane / TS, ox = (int)lane % TS;
  const uint32_t pix_bytes = (uint32_t)p.C * io::kBytes;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;  // < 2^24 (checked at launch)
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(p.output, p.pg_total * (uint32_t)(CG * io::kBytes));
  const float s = p.scale;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)lds;

  // Zero blocks of both buffers (DMA tails only ever write zeros there).
  for (int z = (int)lane * 16; z < BUF - ZERO; z += kPipeThreads * 16) {
    *reinterpret_cast<uint4 *>(lds + ZERO + z) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4 *>(lds + BUF + ZERO + z) = make_uint4(0, 0, 0, 0);
  }

  // DMA slot u of this wave is block q = wave + WAVES u, lane wl's chunk
  // ci = 64 q + wl = (window pixel ci / NCH, chunk ci % NCH).  Its window
  // coordinates are the same for every item: packed once.
  uint32_t dpk[SLOTS];
#pragma unroll
  for (int u = 0; u < SLOTS; ++u) {
    const int q = (int)wave + WAVES * u;
    const int ci = q * 64 + (int)wl;
    const int idx = ci / NCH, ch = ci % NCH;
    const int sy = idx / SPAN_W, sx = idx - sy * SPAN_W;
    dpk[u] = (q < NDMA && idx < SPAN) ? ((uint32_t)sy << 8 | (uint32_t)sx | (uint32_t)ch << 16) : 0xFFFFFFFFu;
  }

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
    const int r0 = (int)tyi * TS, c0 = (int)txi * TS;
    I.Y0 = r0 - p.PH - R;  // window origin (stride and dilation 1)
    I.X0 = c0 - p.PW - R;
    I.ho = r0 + oy;
    I.wo = c0 + ox;
    I.live = I.ho < p.Ho && I.wo < p.Wo;
    I.pg = I.live ? (((I.n * (uint32_t)p.Ho + I.ho) * (uint32_t)p.Wo + I.wo) * (uint32_t)p.G) + I.g : 0u;
    return I;
  };

  // Stream pass h of item I's window into buffer b.
  auto issue_window = [&](const Item &I, int h, int b) {
    const uint32_t base = I.n * (uint32_t)p.H * row_bytes + (I.g * CG + h * CPP) * io::kBytes;
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      const int q = (int)wave + WAVES * u;
      if (q < NDMA) {  // wave-uniform
        const uint32_t pk = dpk[u];
        const int gy = I.Y0 + (int)((pk >> 8) & 0xFFu), gx = I.X0 + (int)(pk & 0xFFu);
        const bool ok = pk != 0xFFFFFFFFu && (uint32_t)gy < (uint32_t)p.H && (uint32_t)gx < (uint32_t)p.W;
        const uint32_t voff = ok ? base + __umul24((uint32_t)gy, row_bytes) + __umul24((uint32_t)gx, pix_bytes) +
                                       ((pk >> 16) & 1u) * CHUNK
                                 : kOutOfRange;
        dma16(rin, __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(b * BUF + q * 1024)), voff);
      }
    }
  };

  // Per-lane chunk rotation (bank spreading) and its byte offsets.
  int rot[NCH];
#pragma unroll
  for (int t = 0; t < NCH; ++t) rot[t] = ((t + (int)lane) % NCH) * CHUNK;

  const XcdWalk walk = xcd_walk(blockIdx.x, gridDim.x, tg.items);
  uint32_t item = walk.first;
  if (item >= walk.end) return;  // block-uniform

  // Prologue: first pass window and the row data of the first item.
  Item cur = decode(item);
  float off[18], msk[9];
  issue_window(cur, 0, 0);
  load_offsets<DT>(p.offset, cur.pg, off);
  load_mask<DT>(p.mask, cur.pg, msk);
  int buf = 0;
  // The previous pass's packed output, stored one pass late.
  uint32_t outw[NCH][4];
  uint32_t out_base = kOutOfRange;
  bool have_out = false;

  struct Pt {
    float w00, w01, w10, w11;
    int A;
  };

  while (true) {
    const uint32_t next = item + walk.stride;
    const bool more = next < walk.end;  // block-uniform
    float off_n[18], msk_n[9];
    Pt P[K];
    uint32_t fbmask = 0;
    // Map coordinates of the top-left corner of points that left the window,
    // packed as two 16-bit values (clamped: a clamped point is outside the
    // map either way), for the global fix-up of every pass.
    uint32_t fbpos[K];

    // The item's row data was requested a pass ago; the compiler's own wait
    // for it lands here, before the first barrier of the item.
    // Modulation scalars, then every point's location, weights and
    // window address, kept for all passes of the item.
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
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = k / 3, j = k % 3;
      const float dx = s * off[2 * k], dy = s * off[2 * k + 1];
      const bool nan_loc = (dx != dx) | (dy != dy);
      const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
      const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
      const float fx = floorf(cx), fy = floorf(cy);
      const float lx = cx - fx, ly = cy - fy;
      const int ty = oy + i + R + (int)fy, tx = ox + j + R + (int)fx;  // window coordinates
      const float mk = nan_loc ? __builtin_nanf("") : m[k];
      const float wy0 = (1.f - ly) * mk, wy1 = ly * mk;
      P[k].w00 = wy0 * (1.f - lx);
      P[k].w01 = wy0 * lx;
      P[k].w10 = wy1 * (1.f - lx);
      P[k].w11 = wy1 * lx;
      const bool inside = !nan_loc && (uint32_t)ty <= (uint32_t)LIM && (uint32_t)tx <= (uint32_t)LIM;
      P[k].A = inside ? ty * ROW + tx * PIXB : ZERO;
      fbmask |= (uint32_t)(cur.live && !inside && !nan_loc) << k;
      const int y0 = min(max(cur.Y0 + ty, -32768), 32767), x0 = min(max(cur.X0 + tx, -32768), 32767);
      fbpos[k] = ((uint32_t)y0 & 0xFFFFu) | ((uint32_t)x0 << 16);
    }

#pragma unroll 1
    for (int h = 0; h < NH; ++h) {
      // This wave's share of the current window (and every older access) has
      // landed once vmcnt drains; the barrier makes that true for all waves
      // and retires every read of the other buffer.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();

      if (h + 1 < NH) {
        issue_window(cur, h + 1, buf ^ 1);
      } else if (more) {
        const Item nx = decode(next);
        issue_window(nx, 0, buf ^ 1);
        load_offsets<DT>(p.offset, nx.pg, off_n);
        load_mask<DT>(p.mask, nx.pg, msk_n);
      }
      if (have_out) {
#pragma unroll
        for (int t = 0; t < NCH; ++t) buffer_store_words<4>(rout, out_base + (uint32_t)rot[t], outw[t]);
      }

      const unsigned char *win = lds + buf * BUF;
      float acc[NCH][CPC];
#pragma unroll
      for (int t = 0; t < NCH; ++t)
#pragma unroll
        for (int c = 0; c < CPC; ++c) acc[t][c] = 0.f;

      auto gather = [&](const Pt &Q, uint32_t (&V)[NCH][4][4]) {
        const unsigned char *src = win + Q.A;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
          const unsigned char *q = src + rot[t];
          lds_read16(q, V[t][0]);
          lds_read16(q + PIXB, V[t][1]);
          lds_read16(q + ROW, V[t][2]);
          lds_read16(q + ROW + PIXB, V[t][3]);
        }
      };
      auto accumulate = [&](const Pt &Q, const uint32_t (&V)[NCH][4][4]) {
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
          float f00[CPC], f01[CPC], f10[CPC], f11[CPC];
          unpack<DT, 4>(V[t][0], f00);
          unpack<DT, 4>(V[t][1], f01);
          unpack<DT, 4>(V[t][2], f10);
          unpack<DT, 4>(V[t][3], f11);
#pragma unroll
          for (int c = 0; c < CPC; ++c) {
            acc[t][c] = fmaf(Q.w00, f00[c], acc[t][c]);
            acc[t][c] = fmaf(Q.w01, f01[c], acc[t][c]);
            acc[t][c] = fmaf(Q.w10, f10[c], acc[t][c]);
            acc[t][c] = fmaf(Q.w11, f11[c], acc[t][c]);
          }
        }
      };

      // The gathers of point k+1 are in flight while point k's FMAs run.
      uint32_t V0[NCH][4][4], V1[NCH][4][4];
      gather(P[0], V0);
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (k + 1 < K) gather(P[k + 1], (k & 1) ? V0 : V1);
        __builtin_amdgcn_sched_barrier(0);
        accumulate(P[k], (k & 1) ? V1 : V0);
      }

      // Points whose corners left the window: global gathers of this pass's
      // channels (rare; a wave skips a point no lane of it needs).
      const uint32_t img = cur.n * (uint32_t)p.H * row_bytes;
      const uint32_t chan = (cur.g * CG + h * CPP) * io::kBytes;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const bool fb = (fbmask >> k) & 1u;
        if (__builtin_amdgcn_ballot_w64(fb) != 0) {
          if (fb) {
            const int y0 = (int)(int16_t)(fbpos[k] & 0xFFFFu), x0 = (int)(int16_t)(fbpos[k] >> 16);
            const bool vy0 = (uint32_t)y0 < (uint32_t)p.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)p.H;
            const bool vx0 = (uint32_t)x0 < (uint32_t)p.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)p.W;
            const uint32_t a00 = img + (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_bytes + chan;
            uint32_t V[NCH][4][4];
#pragma unroll
            for (int t = 0; t < NCH; ++t) {
              const uint32_t ct = (uint32_t)rot[t];
              buffer_load_words<4>(rin, (vy0 && vx0) ? a00 + ct : kOutOfRange, V[t][0]);
              buffer_load_words<4>(rin, (vy0 && vx1) ? a00 + pix_bytes + ct : kOutOfRange, V[t][1]);
              buffer_load_words<4>(rin, (vy1 && vx0) ? a00 + row_bytes + ct : kOutOfRange, V[t][2]);
              buffer_load_words<4>(rin, (vy1 && vx1) ? a00 + row_bytes + pix_bytes + ct : kOutOfRange, V[t][3]);
            }
            accumulate(P[k], V);
          }
        }
      }

      // acc[t] holds the chunk at byte offset rot[t] of this pass's slice; a
      // dead lane's store carries an out-of-range offset and is dropped.
      out_base = cur.live ? cur.pg * (uint32_t)(CG * io::kBytes) + (uint32_t)(h * PIXB) : kOutOfRange;
#pragma unroll
      for (int t = 0; t < NCH; ++t) pack_words<DT, CPC>(acc[t], outw[t]);
      have_out = true;
      buf ^= 1;
    }

    if (!more) break;
    item = next;
    cur = decode(item);
#pragma unroll
    for (int q = 0; q < 18; ++q) off[q] = off_n[q];
#pragma unroll
    for (int q = 0; q < 9; ++q) msk[q] = msk_n[q];
  }
#pragma unroll
  for (int t = 0; t < NCH; ++t) buffer_store_words<4>(rout, out_base + (uint32_t)rot[t], outw[t]);
}

namespace {

template <int DT, bool SM>
hipError_t launch_pipe(const FwdParams &p, const TileGeom &tg, hipStream_t s) {
  auto kern = dcn_fwd_pipe_kernel<DT, SM>;
  const size_t lds = 2 * (size_t)kPipeBuf;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const uint32_t blocks = std::min<uint32_t>(tg.items, (uint32_t)kPipeBlocksPerCu * (uint32_t)cus);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kPipeThreads), lds, s, p, tg);
  return hipGetLastError();
}

}  // namespace

// Stride 1, dilation 1, 3x3 points, rows below 16 MB (24-bit offset
// products); hipErrorNotSupported otherwise.
hipError_t launch_forward_pipe(int dtype, int softmax, const FwdParams &p, hipStream_t s) {
  if (p.KH != 3 || p.KW != 3 || p.SH != 1 || p.SW != 1 || p.DH != 1 || p.DW != 1)
    return hipErrorNotSupported;
  const int64_t row_bytes = (int64_t)p.W * p.C * (dtype == DCN_F32 ? 4 : 2);
  if (row_bytes >= (int64_t(1) << 24)) return hipErrorNotSupported;
  TileGeom tg{};
  tg.span_h = tg.span_w = kPipeSpan;
  const int tiles_y = (p.Ho + kPipeTile - 1) / kPipeTile;
  tg.tiles_x = (p.Wo + kPipeTile - 1) / kPipeTile;
  tg.tiles_per_img = tiles_y * tg.tiles_x;
  const int64_t imgs = p.pg_total / ((int64_t)p.Ho * p.Wo * p.G);
  const int64_t items = imgs * tg.tiles_per_img * p.G;
  if (items <= 0 || items >= (int64_t(1) << 31)) return hipErrorNotSupported;
  tg.items = (uint32_t)items;
  tg.div_g = make_fast_div((uint32_t)p.G);
  tg.div_tiles = make_fast_div((uint32_t)tg.tiles_per_img);
  tg.div_tiles_x = make_fast_div((uint32_t)tg.tiles_x);
  tg.div_span_w = make_fast_div((uint32_t)tg.span_w);
  switch (dtype) {
    case DCN_F32: return softmax ? launch_pipe<DCN_F32, true>(p, tg, s) : launch_pipe<DCN_F32, false>(p, tg, s);
    case DCN_F16: return softmax ? launch_pipe<DCN_F16, true>(p, tg, s) : launch_pipe<DCN_F16, false>(p, tg, s);
    case DCN_BF16: return softmax ? launch_pipe<DCN_BF16, true>(p, tg, s) : launch_pipe<DCN_BF16, false>(p, tg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dcn
