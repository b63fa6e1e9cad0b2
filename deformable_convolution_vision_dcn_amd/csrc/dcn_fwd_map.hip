// dcn_fwd_map.hip -- whole-map gfx950 forward kernel of the DCN core for 3x3
// kernel points on small feature maps (wmrh.cn/news/61976, section 二 steps
// 2-4 and section 三; the late InternImage stages run at 24x24 and 12x12),
// all nine or the eight left by DCNv4's remove_center
// (pnsm.cn/news/2029644.html section 3.3).
//
// Why a second layout: a 16x16 output tile on a 24x24 or 12x12 map leaves up
// to 44 % of the lanes of the tiled kernels without a pixel, and its window
// (tile plus halo) re-reads most of the map for every tile.  Here a work item
// is (image, block of GPI groups) and the whole map of each of those groups,
// with a one-pixel zero border, sits in LDS: every lane owns a pixel-group,
// every sample reads LDS (a sample whose top-left corner lies outside the
// bordered map touches no map pixel and reads a zero block), and there is no
// global fix-up path at all.
//
// Block = 192 threads (3 waves), several blocks per CU.  The windows arrive
// by direct global->LDS loads (buffer_load_dwordx4 ... lds: lane l's 16
// bytes land at the wave's LDS address + 16 l), so no VGPRs hold them; while one block waits for
// its window the other blocks of the CU compute.  Lane j of pass q owns
// pixel-group index q * 192 + j of the item, groups fastest, so neighbouring
// lanes read neighbouring offset and mask rows.
//
// LDS: group window gl at gl * GS, bordered pixel (y + 1, x + 1) at
// (y + 1) * WROW + (x + 1) * PIXB, PIXB = one pixel's 16 channels; then a
// zero block of one row plus two pixels.  A lane reads the 16-byte chunks of
// a corner in the rotated order (t + lane) mod NCH to spread banks.
#include <algorithm>

#include "dcn_device.hpp"
#include "dcn_launch.hpp"

namespace dcn {

#ifndef DCN_MAP_WAVES
#define DCN_MAP_WAVES 4
#endif
constexpr int kMapThreads = 192;
// Waves per SIMD the register budget must allow (128 VGPRs).
template <int DT>
constexpr int map_waves() { return DCN_MAP_WAVES; }
constexpr int kMapMaxLds = 48 * 1024;  // window budget per block (3+ blocks per CU)

template <int DT>
constexpr int map_pixb() { return DT == DCN_F32 ? 64 : 32; }

struct MapGeom {
  int32_t gpi_log2;      // groups per item = 1 << gpi_log2
  int32_t wrow;          // LDS bytes per bordered window row: (W + 2) * PIXB
  int32_t gstride;       // LDS bytes per group window: (H + 2) * wrow
  int32_t zero;          // LDS offset of the zero block
  int32_t units;         // 16-byte window units of one item
  int32_t passes;        // passes of 192 pixel-groups per item
  uint32_t pgi;          // pixel-groups per item: GPI * Ho * Wo
  uint32_t items;        // (image, group block) work items
  uint32_t gblocks;      // group blocks per image: ceil(G / GPI)
  FastDiv div_gblocks, div_wo, div_ww, div_cell;
};

namespace {

// 64 lanes x 16 bytes from the buffer resource into LDS at dst (wave
// uniform) + 16 * lane; an out-of-range voff writes zeros.
__device__ __forceinline__ void map_dma16(__amdgpu_buffer_rsrc_t r, unsigned char *dst, uint32_t voff) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, voff, 0, 0, 0);
}

}  // namespace

// RC: the centre point is removed (8 points; point k sits at grid index
// k + (k >= 4)).
template <int DT, bool SOFTMAX, bool RC>
__global__ void __launch_bounds__(kMapThreads, map_waves<DT>()) dcn_fwd_map_kernel(FwdParams p, MapGeom mg) {
  using io = Io<DT>;
  constexpr int CG = kGroupChannels;
  constexpr int PIXB = map_pixb<DT>();
  constexpr int CHUNK = 16;
  constexpr int NCH = PIXB / CHUNK;        // 16-byte chunks per pixel slice: 4 or 2
  constexpr int CPC = CHUNK / io::kBytes;  // channels per chunk: 4 or 8
  constexpr int GB = CG * io::kBytes;      // bytes of one group of one pixel
  constexpr int K = RC ? 8 : 9;

  extern __shared__ __align__(16) unsigned char lds[];

  const uint32_t lane = threadIdx.x;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(lane / 64);
  const uint32_t wl = lane % 64;
  const uint32_t pix_bytes = (uint32_t)p.C * io::kBytes;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const uint32_t img_bytes = (uint32_t)p.H * row_bytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const __amdgpu_buffer_rsrc_t roff = make_rsrc(p.offset, p.off_bytes);
  const __amdgpu_buffer_rsrc_t rmask = make_rsrc(p.mask, p.mask_bytes);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(p.output, p.out_bytes);
  const uint32_t gmask = (1u << mg.gpi_log2) - 1u;
  const uint32_t ncell = (uint32_t)(p.H + 2) * (uint32_t)(p.W + 2);
  const float s = p.scale;

  // Zero block (the barrier that publishes the windows orders it).
  for (int z = (int)lane * 16; z < mg.wrow + 2 * PIXB; z += kMapThreads * 16)
    *reinterpret_cast<uint4 *>(lds + mg.zero + z) = make_uint4(0, 0, 0, 0);

  // Per-lane chunk rotation (bank spreading), as byte offsets.
  uint32_t rot[NCH];
#pragma unroll
  for (int t = 0; t < NCH; ++t) rot[t] = ((t + lane) % NCH) * CHUNK;

  struct Pg {
    uint32_t pg, gl;
    int by, bx;  // bordered window coordinates of the point (0, 0) before its offset
    bool live;
  };
  auto pixel_group = [&](uint32_t n, uint32_t g0, int q) {
    Pg r;
    const uint32_t j = (uint32_t)q * kMapThreads + lane;
    r.gl = j & gmask;
    const uint32_t pix = j >> mg.gpi_log2;
    const uint32_t ho = fast_div(pix, mg.div_wo), wo = pix - ho * (uint32_t)p.Wo;
    const uint32_t g = g0 + r.gl;
    r.live = j < mg.pgi && g < (uint32_t)p.G;
    r.pg = r.live ? ((n * (uint32_t)p.Ho + ho) * (uint32_t)p.Wo + wo) * (uint32_t)p.G + g : 0u;
    r.by = (int)ho * p.SH - p.PH + 1;
    r.bx = (int)wo * p.SW - p.PW + 1;
    return r;
  };

  RowWords<DT, K> rw[2];

  // One work item per block: nothing is carried from item to item, and the
  // hardware then starts each block as soon as a slot frees up, so the last
  // items do not wait behind a fixed assignment.
  {
    const uint32_t item = blockIdx.x;
    const uint32_t n = fast_div(item, mg.div_gblocks);
    const uint32_t g0 = (item - n * mg.gblocks) << mg.gpi_log2;

    // Windows of the item's groups: unit e = cell * NCH + chunk, cell =
    // (gl, wy, wx) of the bordered map; units past the end (and border or
    // missing-group cells) read as zeros.
    const uint32_t img = n * img_bytes;
    for (uint32_t e0 = wave * 64u; e0 < (uint32_t)mg.units; e0 += kMapThreads) {
      const uint32_t e = e0 + wl;
      const uint32_t cell = e / NCH, chunk = e % NCH;
      const uint32_t gl = fast_div(cell, mg.div_cell);
      const uint32_t rem = cell - gl * ncell;
      const uint32_t wy = fast_div(rem, mg.div_ww), wx = rem - wy * (uint32_t)(p.W + 2);
      const uint32_t y = wy - 1u, x = wx - 1u, g = g0 + gl;
      const bool ok = y < (uint32_t)p.H && x < (uint32_t)p.W && gl <= gmask && g < (uint32_t)p.G;
      const uint32_t off = ok ? img + y * row_bytes + x * pix_bytes + g * GB + chunk * CHUNK : kOutOfRange;
      map_dma16(rin, lds + e0 * 16u, off);
    }
    {
      const Pg q0 = pixel_group(n, g0, 0);
      load_row_words<DT, K>(roff, rmask, q0.pg, rw[0]);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's window loads have landed
    __syncthreads();                     // the windows are in LDS

    // One pass: decode this pass's rows from (cw, cm), request the next
    // pass's into (nw, nm), then the nine samples of every lane's pixel-group.
    auto pass = [&](int q, const RowWords<DT, K> &cr, RowWords<DT, K> &nr) {
      const Pg cur = pixel_group(n, g0, q);
      float off[2 * K], msk[K];
      decode_row_words<DT, K>(cur.pg, cr, off, msk);
      if (q + 1 < mg.passes) load_row_words<DT, K>(roff, rmask, pixel_group(n, g0, q + 1).pg, nr);
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

      const uint32_t gbase = cur.gl * (uint32_t)mg.gstride;
      // Point k: its weights (modulation folded in) and LDS address.
      struct Pt {
        float w00, w01, w10, w11;
        uint32_t A;
      };
      auto locate = [&](int k, Pt &P) {
        const int g3 = RC ? k + (k >= 4) : k;  // grid index
        const int i = g3 / 3, j = g3 % 3;
        const float dx = s * off[2 * k], dy = s * off[2 * k + 1];
        const bool nan_loc = (dx != dx) | (dy != dy);
        const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
        const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
        const float fx = floorf(cx), fy = floorf(cy);
        const float lx = cx - fx, ly = cy - fy;
        // bordered window coordinates of the top-left corner
        const int ty = cur.by + i * p.DH + (int)fy, tx = cur.bx + j * p.DW + (int)fx;
        const float mk = nan_loc ? __builtin_nanf("") : m[k];
        const float wy1 = ly * mk, wy0 = mk - wy1;
        P.w01 = wy0 * lx;
        P.w00 = wy0 - P.w01;
        P.w11 = wy1 * lx;
        P.w10 = wy1 - P.w11;
        const bool inside = !nan_loc && (uint32_t)ty <= (uint32_t)p.H && (uint32_t)tx <= (uint32_t)p.W;
        P.A = inside ? gbase + (uint32_t)ty * (uint32_t)mg.wrow + (uint32_t)tx * PIXB : (uint32_t)mg.zero;
      };
      // The four corners of chunk t of a point, then their FMAs.
      auto fetch = [&](const Pt &P, int t, uint32_t (&q)[4][4]) {
        const unsigned char *c = lds + P.A + rot[t];
        const unsigned char *corner[4] = {c, c + PIXB, c + mg.wrow, c + mg.wrow + PIXB};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint4 v = *reinterpret_cast<const uint4 *>(corner[r]);
          q[r][0] = v.x;
          q[r][1] = v.y;
          q[r][2] = v.z;
          q[r][3] = v.w;
        }
      };
      auto consume = [&](const Pt &P, int t, const uint32_t (&q)[4][4]) {
        float f00[CPC], f01[CPC], f10[CPC], f11[CPC];
        unpack<DT, 4>(q[0], f00);
        unpack<DT, 4>(q[1], f01);
        unpack<DT, 4>(q[2], f10);
        unpack<DT, 4>(q[3], f11);
#pragma unroll
        for (int c2 = 0; c2 < CPC; ++c2) {
          acc[t][c2] = fmaf(P.w00, f00[c2], acc[t][c2]);
          acc[t][c2] = fmaf(P.w01, f01[c2], acc[t][c2]);
          acc[t][c2] = fmaf(P.w10, f10[c2], acc[t][c2]);
          acc[t][c2] = fmaf(P.w11, f11[c2], acc[t][c2]);
        }
        // Pin the chunk's sums here: otherwise the compiler sinks every FMA
        // of the pass to its end and keeps all nine points' corners live.
        pin_values(acc[t]);
      };
      // Software pipeline over the K * NCH (point, chunk) steps: the corners
      // of step u + 1 are requested before step u's arithmetic, so one
      // step's LDS latency overlaps the previous step's FMAs within the wave.
      // Two register sets alternate (static after unrolling).
      constexpr int STEPS = K * NCH;
      Pt pts[2];
      uint32_t qa[4][4], qb[4][4];
      locate(0, pts[0]);
      fetch(pts[0], 0, qa);
#pragma unroll
      for (int u = 0; u < STEPS; ++u) {
        const int k = u / NCH, t = u % NCH;
        if (u + 1 < STEPS) {
          const int k1 = (u + 1) / NCH, t1 = (u + 1) % NCH;
          if (t1 == 0) locate(k1, pts[k1 & 1]);
          fetch(pts[k1 & 1], t1, (u & 1) ? qa : qb);
        }
        consume(pts[k & 1], t, (u & 1) ? qb : qa);
      }

      // acc[t] holds the chunk at byte offset rot[t] of the 16-channel slice;
      // a dead lane's store carries an out-of-range offset and is dropped.
      const uint32_t obase = cur.live ? cur.pg * (uint32_t)GB : kOutOfRange;
#pragma unroll
      for (int t = 0; t < NCH; ++t) {
        uint32_t w[4];
        pack_words<DT, CPC>(acc[t], w);
        buffer_store_words_aux<4, kNonTemporal>(rout, obase + rot[t], w);
      }
    };
#pragma unroll 1
    for (int q = 0; q < mg.passes; ++q) {
      pass(q, rw[0], rw[1]);
      rw[0] = rw[1];
    }
  }
}

namespace {

template <int DT, bool SM, bool RC>
hipError_t launch_map(const FwdParams &p, const MapGeom &mg, size_t lds, hipStream_t s) {
  auto kern = dcn_fwd_map_kernel<DT, SM, RC>;
  const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(mg.items), dim3(kMapThreads), lds, s, p, mg);
  return hipGetLastError();
}

template <bool RC>
hipError_t launch_map_dt(int dtype, int softmax, const FwdParams &p, const MapGeom &mg, size_t lds, hipStream_t s) {
  switch (dtype) {
    case DCN_F32: return softmax ? launch_map<DCN_F32, true, RC>(p, mg, lds, s) : launch_map<DCN_F32, false, RC>(p, mg, lds, s);
    case DCN_F16: return softmax ? launch_map<DCN_F16, true, RC>(p, mg, lds, s) : launch_map<DCN_F16, false, RC>(p, mg, lds, s);
    case DCN_BF16: return softmax ? launch_map<DCN_BF16, true, RC>(p, mg, lds, s) : launch_map<DCN_BF16, false, RC>(p, mg, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// 3x3 points (nine, or eight without the centre) on a map whose bordered
// window (of at least one group) fits the LDS budget; hipErrorNotSupported (nothing launched) otherwise.  Groups
// per item: the smallest power of two that keeps the passes' lanes at least
// 90 % busy, within the budget (else the best one found).
hipError_t launch_forward_map(int dtype, int softmax, const FwdParams &p, hipStream_t s) {
  if (p.KH != 3 || p.KW != 3) return hipErrorNotSupported;
  const int pixb = dtype == DCN_F32 ? 64 : 32;
  const int64_t cell_bytes = (int64_t)(p.H + 2) * (p.W + 2) * pixb;
  const int64_t howo = (int64_t)p.Ho * p.Wo;
  const int64_t imgs = p.pg_total / (howo * p.G);
  int best = -1;
  double best_use = 0.0;
  for (int l = 0; (1 << l) <= 16 && (1 << (l > 0 ? l - 1 : 0)) < p.G; ++l) {
    const int64_t gpi = int64_t(1) << l;
    if (gpi * cell_bytes > kMapMaxLds) break;
    const int64_t pgi = gpi * howo;
    const int64_t passes = (pgi + kMapThreads - 1) / kMapThreads;
    const double use = (double)(std::min<int64_t>(gpi, p.G) * howo) / (double)(passes * kMapThreads);
    if (use > best_use + 1e-9) {
      best_use = use;
      best = l;
    }
    if (use >= 0.9) break;
  }
  if (best < 0) return hipErrorNotSupported;
  MapGeom mg{};
  mg.gpi_log2 = best;
  const int64_t gpi = int64_t(1) << best;
  mg.wrow = (p.W + 2) * pixb;
  mg.gstride = (int32_t)cell_bytes;
  const int64_t units = gpi * cell_bytes / 16;
  mg.units = (int32_t)units;
  mg.zero = (int32_t)((units + 63) / 64 * 1024);  // after the last 1 KB DMA block
  mg.pgi = (uint32_t)(gpi * howo);
  mg.passes = (int32_t)((mg.pgi + kMapThreads - 1) / kMapThreads);
  mg.gblocks = (uint32_t)((p.G + gpi - 1) / gpi);
  const int64_t items = imgs * mg.gblocks;
  if (items <= 0 || items >= (int64_t(1) << 31)) return hipErrorNotSupported;
  mg.items = (uint32_t)items;
  mg.div_gblocks = make_fast_div(mg.gblocks);
  mg.div_wo = make_fast_div((uint32_t)p.Wo);
  mg.div_ww = make_fast_div((uint32_t)(p.W + 2));
  mg.div_cell = make_fast_div((uint32_t)((p.H + 2) * (p.W + 2)));
  const size_t lds = (size_t)mg.zero + mg.wrow + 2 * pixb;
  return p.RC ? launch_map_dt<true>(dtype, softmax, p, mg, lds, s) : launch_map_dt<false>(dtype, softmax, p, mg, lds, s);
}

}  // namespace dcn
