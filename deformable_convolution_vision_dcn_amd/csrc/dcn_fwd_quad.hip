// dcn_fwd_quad.hip -- double-buffered LDS-tiled gfx950 forward kernel of the
// DCN core for 3x3 kernel points (wmrh.cn/news/61976, section 二 steps 2-4
// and section 三).
//
// Block = 1024 threads = 256 lane-quads = one 16x16 output tile of one group
// (one work item) per step; one block per CU (16 waves, 4 per SIMD), walking
// its XCD's range of (image, tile, group) items.
//
// Per pixel-group one quad: lane `sub` owns channels [4 sub, 4 sub + 4) and
// computes the location, bilinear weights (modulation folded in) and LDS
// address of the kernel points k = sub, sub + 4, sub + 8; DPP quad
// broadcasts hand them to the other three lanes.  Each lane reads its chunk
// of the four corners and does 4 FMAs per channel per point.  The softmax
// over the nine logits is a quad reduction.
//
// Pipeline: two LDS window buffers.  While item i is computed from one, the
// window of item i+1 (its regular 3x3 footprint plus a halo of R pixels,
// zero outside the map) streams into the other with direct global->LDS
// loads (lane l's 16 bytes land at M0 + 16 l), and its offsets and logits
// stream into registers.  One barrier per item.  The DMA is issued from
// inline asm so that the compiler does not wait for it before reading the
// other buffer; it is waited for explicitly before the barrier.  The output
// of item i is stored after that barrier, so the wait never covers fresh
// stores.
//
// Samples whose corners leave the window read a zero block on the main path
// and are fixed up from global memory after the window work of the item (so
// that their waits find the next window's DMA complete); the buffer range
// check reads 0 for corners outside the map.
#include <algorithm>
#include <type_traits>

#include "dcn_device.hpp"

namespace dcn {

constexpr int kQuadThreads = 1024;
constexpr int kQuadTile = 16;
constexpr int kQuadHalo = 7;

template <int DT>
constexpr int quad_pixb() { return DT == DCN_F32 ? 64 : 32; }

namespace {

template <int O>
__device__ __forceinline__ int qb(int v) {
  constexpr int ctrl = O | (O << 2) | (O << 4) | (O << 6);  // quad_perm [O,O,O,O]
  return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, false);
}
template <int O>
__device__ __forceinline__ float qb(float v) {
  return __int_as_float(qb<O>(__float_as_int(v)));
}
__device__ __forceinline__ float qmax(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ float qsum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  return v;
}

template <int NW>
__device__ __forceinline__ void lds_get(const unsigned char *src, uint32_t (&w)[NW]) {
  if constexpr (NW == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(src);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2 *>(src);
    w[0] = v.x; w[1] = v.y;
  }
}

template <int DT>
__device__ __forceinline__ float2 get_pair(const void *base, uint32_t e) {
  if constexpr (DT == DCN_F32) {
    return static_cast<const float2 *>(base)[e];
  } else {
    const uint32_t w = static_cast<const uint32_t *>(base)[e];
    return make_float2(Io<DT>::lo(w), Io<DT>::hi(w));
  }
}
template <int DT>
__device__ __forceinline__ float get_one(const void *base, uint32_t e) {
  if constexpr (DT == DCN_F32) {
    return static_cast<const float *>(base)[e];
  } else if constexpr (DT == DCN_F16) {
    return (float)static_cast<const _Float16 *>(base)[e];
  } else {
    return __uint_as_float((uint32_t) static_cast<const uint16_t *>(base)[e] << 16);
  }
}

// 64 lanes x 16 bytes into LDS at lds_base (wave uniform) + 16 * lane; an
// out-of-range voff writes zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(r)
               : "memory");
}

}  // namespace

// Geometry of one launch of the kernel below.
struct QuadGeom {
  TileGeom t;
  int32_t buf_bytes;  // one window buffer incl. its zero block, multiple of 1 KB
  int32_t ndma;       // 1 KB DMA blocks per window
};

template <int DT, bool SOFTMAX>
__global__ void __launch_bounds__(kQuadThreads) dcn_fwd_quad_kernel(FwdParams p, QuadGeom qg) {
  using io = Io<DT>;
  constexpr int CG = kGroupChannels;
  constexpr int CPL = 4;                     // channels per lane
  constexpr int NW = CPL * io::kBytes / 4;   // words per lane per corner
  constexpr int LANE_BYTES = CPL * io::kBytes;
  constexpr int PIXB = quad_pixb<DT>();
  constexpr int NCH = PIXB / 16;             // 16-byte DMA chunks per pixel slice
  constexpr int TS = kQuadTile, R = kQuadHalo, K = 9;
  const TileGeom &tg = qg.t;

  extern __shared__ __align__(16) unsigned char lds[];

  const uint32_t tid = threadIdx.x;
  const uint32_t quad = tid >> 2, sub = tid & 3;
  const uint32_t wl = tid & 63, wave = tid >> 6;
  const int oy = (int)quad / TS, ox = (int)quad % TS;
  const uint32_t pix_bytes = (uint32_t)p.C * io::kBytes;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const __amdgpu_buffer_rsrc_t rout = make_rsrc(p.output, p.pg_total * (uint32_t)(CG * io::kBytes));
  const int span_w = tg.span_w;
  const int span = tg.span_h * span_w;
  const int row_lds = span_w * PIXB;
  const int zero_off = span * PIXB;
  const int lim_y = tg.span_h - 2, lim_x = span_w - 2;
  const int BUF = qg.buf_bytes;
  const float s = p.scale;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)lds;

  // Zero blocks of both buffers (DMA tails only ever write zeros there).
  for (int z = zero_off + (int)tid * 16; z < BUF; z += kQuadThreads * 16) {
    *reinterpret_cast<uint4 *>(lds + z) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4 *>(lds + BUF + z) = make_uint4(0, 0, 0, 0);
  }

  struct Item {
    uint32_t g, n, img, chan, pg;
    int Y0, X0, ho, wo;
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
    const int r0 = (int)tyi * TS, c0 = (int)txi * TS;
    I.Y0 = r0 * p.SH - p.PH - R;  // window origin in input coordinates
    I.X0 = c0 * p.SW - p.PW - R;
    I.img = I.n * (uint32_t)p.H * row_bytes;
    I.chan = (I.g * CG + sub * CPL) * io::kBytes;
    I.ho = r0 + oy;
    I.wo = c0 + ox;
    I.live = I.ho < p.Ho && I.wo < p.Wo;
    I.pg = I.live ? (((I.n * (uint32_t)p.Ho + I.ho) * (uint32_t)p.Wo + I.wo) * (uint32_t)p.G) + I.g : 0u;
    return I;
  };

  // Window of item I into buffer b: this wave takes DMA blocks wave,
  // wave + 16, ...; block q covers window chunks [64 q, 64 q + 64).
  auto issue_window = [&](const Item &I, int b) {
    const uint32_t base = I.img + (I.g * CG) * io::kBytes;
    for (int q = (int)wave; q < qg.ndma; q += kQuadThreads / 64) {
      const uint32_t ci = (uint32_t)q * 64 + wl;
      const uint32_t idx = ci / NCH, ch = ci % NCH;
      const uint32_t sy = fast_div(idx, tg.div_span_w);
      const uint32_t sx = idx - sy * (uint32_t)span_w;
      const int gy = I.Y0 + (int)sy, gx = I.X0 + (int)sx;
      const bool ok = (int)idx < span && (uint32_t)gy < (uint32_t)p.H && (uint32_t)gx < (uint32_t)p.W;
      const uint32_t voff = ok ? base + (uint32_t)gy * row_bytes + (uint32_t)gx * pix_bytes + ch * 16u : kOutOfRange;
      dma16(rin, __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(b * BUF + q * 1024)), voff);
    }
  };

  // Own points k = sub + 4 r: offsets and logits.
  auto load_rows = [&](const Item &I, float2 (&o)[3], float (&l)[3]) {
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int k = (int)sub + 4 * r;
      const int kk = k < K ? k : 0;
      o[r] = get_pair<DT>(p.offset, I.pg * K + kk);
      l[r] = get_one<DT>(p.mask, I.pg * K + kk);
    }
  };

  const XcdWalk walk = xcd_walk(blockIdx.x, gridDim.x, tg.items);
  uint32_t item = walk.first;
  if (item >= walk.end) return;  // block-uniform

  Item cur = decode(item);
  float2 off[3];
  float lg[3];
  issue_window(cur, 0);
  load_rows(cur, off, lg);
  int buf = 0;
  uint32_t outw[NW];
  uint32_t out_off = kOutOfRange;
  bool have_out = false;

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  while (true) {
    __builtin_amdgcn_s_waitcnt(0);  // own DMA share and row loads of this item
    __syncthreads();                // everyone's share; the other buffer is free

    const uint32_t next = item + walk.stride;
    const bool more = next < walk.end;  // block-uniform
    float2 off_n[3];
    float lg_n[3];
    if (more) {
      // (decoded again after the compute; nothing of it is kept meanwhile)
      const Item nx = decode(next);
      issue_window(nx, buf ^ 1);
      load_rows(nx, off_n, lg_n);
    }
    if (have_out) {
      if constexpr (NW == 4) {
        typedef uint32_t v4 __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(v4{outw[0], outw[1], outw[2], outw[3]}, rout, (int)out_off, 0, 0);
      } else {
        typedef uint32_t v2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(v2{outw[0], outw[1]}, rout, (int)out_off, 0, 0);
      }
    }

    const unsigned char *win = lds + buf * BUF;
    // modulation scalars of the own points
    float m[3];
    if constexpr (SOFTMAX) {
      float l0 = lg[0], l1 = lg[1], l2 = (int)sub + 8 < K ? lg[2] : -INFINITY;
      const float mx = qmax(fmaxf(fmaxf(l0, l1), l2));
      const float e0 = __expf(l0 - mx), e1 = __expf(l1 - mx), e2 = (int)sub + 8 < K ? __expf(l2 - mx) : 0.f;
      const float inv = __builtin_amdgcn_rcpf(qsum(e0 + e1 + e2));
      m[0] = e0 * inv;
      m[1] = e1 * inv;
      m[2] = e2 * inv;
    } else {
      m[0] = lg[0];
      m[1] = lg[1];
      m[2] = lg[2];
    }

    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    uint32_t fbmask = 0;  // own rounds whose point left the window

    // Round r: every lane prepares its own point k = sub + 4r, then the quad
    // consumes the round's points one owner at a time.  A run-time loop with
    // the per-round inputs rotating through scalars keeps one round's state
    // live at a time.
    float2 o2 = off[0], o2n = off[1], o2nn = off[2];
    float mk_ = m[0], mkn = m[1], mknn = m[2];
#pragma unroll 1
    for (int r = 0; r < 3; ++r) {
      const int k = (int)sub + 4 * r;
      const int i = k >= 6 ? 2 : (k >= 3 ? 1 : 0);
      const int j = k - 3 * i;
      const float dx = s * o2.x, dy = s * o2.y;
      const bool nan_loc = (dx != dx) | (dy != dy);
      const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
      const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
      const float fx = floorf(cx), fy = floorf(cy);
      const float lx = cx - fx, ly = cy - fy;
      const int x0 = cur.wo * p.SW - p.PW + j * p.DW + (int)fx;
      const int y0 = cur.ho * p.SH - p.PH + i * p.DH + (int)fy;
      const float mk = nan_loc ? __builtin_nanf("") : mk_;
      const float wy0 = (1.f - ly) * mk, wy1 = ly * mk;
      const float W0 = wy0 * (1.f - lx), W1 = wy0 * lx;
      const float W2 = wy1 * (1.f - lx), W3 = wy1 * lx;
      const int ty = y0 - cur.Y0, tx = x0 - cur.X0;
      const bool inside = !nan_loc && (uint32_t)ty <= (uint32_t)lim_y && (uint32_t)tx <= (uint32_t)lim_x;
      const int A = inside ? ty * row_lds + tx * PIXB : zero_off;
      const bool fb = cur.live && k < K && !inside && !nan_loc &&
                      (uint32_t)(y0 + 1) <= (uint32_t)p.H && (uint32_t)(x0 + 1) <= (uint32_t)p.W;
      fbmask |= (uint32_t)fb << r;

      auto point = [&](auto o_tag) {
        constexpr int O = decltype(o_tag)::value;
        const int a = qb<O>(A);
        const float w00 = qb<O>(W0), w01 = qb<O>(W1);
        const float w10 = qb<O>(W2), w11 = qb<O>(W3);
        uint32_t q00[NW], q01[NW], q10[NW], q11[NW];
        const unsigned char *src = win + a + sub * LANE_BYTES;
        lds_get<NW>(src, q00);
        lds_get<NW>(src + PIXB, q01);
        lds_get<NW>(src + row_lds, q10);
        lds_get<NW>(src + row_lds + PIXB, q11);
        float v00[CPL], v01[CPL], v10[CPL], v11[CPL];
        unpack<DT, NW>(q00, v00);
        unpack<DT, NW>(q01, v01);
        unpack<DT, NW>(q10, v10);
        unpack<DT, NW>(q11, v11);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          acc[c] = fmaf(w00, v00[c], acc[c]);
          acc[c] = fmaf(w01, v01[c], acc[c]);
          acc[c] = fmaf(w10, v10[c], acc[c]);
          acc[c] = fmaf(w11, v11[c], acc[c]);
        }
      };
      point(I0{});
      if (r < 2) {  // the last round holds only k = 8 (owner lane 0)
        point(I1{});
        point(I2{});
        point(I3{});
      }
      o2 = o2n;
      o2n = o2nn;
      mk_ = mkn;
      mkn = mknn;
    }

    // Deferred fix-up of points that left the window: the owner lane
    // recomputes its point; the quad gathers the corners from global memory.
    auto fix_round = [&](auto r_tag) {
      constexpr int r = decltype(r_tag)::value;
      const bool own_fb = (fbmask >> r) & 1u;
      if (__builtin_amdgcn_ballot_w64(own_fb) == 0) return;  // wave-uniform
      const int k = (int)sub + 4 * r;
      const int i = k >= 6 ? 2 : (k >= 3 ? 1 : 0);
      const int j = k - 3 * i;
      const float dx = s * off[r].x, dy = s * off[r].y;
      const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
      const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
      const float fx = floorf(cx), fy = floorf(cy);
      const float lx = cx - fx, ly = cy - fy;
      const int x0 = cur.wo * p.SW - p.PW + j * p.DW + (int)fx;
      const int y0 = cur.ho * p.SH - p.PH + i * p.DH + (int)fy;
      const float wy0 = (1.f - ly) * m[r], wy1 = ly * m[r];
      const float W0 = wy0 * (1.f - lx), W1 = wy0 * lx;
      const float W2 = wy1 * (1.f - lx), W3 = wy1 * lx;
      auto fix = [&](auto o_tag) {
        constexpr int O = decltype(o_tag)::value;
        if (!qb<O>((int)own_fb)) return;
        const float w00 = qb<O>(W0), w01 = qb<O>(W1);
        const float w10 = qb<O>(W2), w11 = qb<O>(W3);
        const int yb = qb<O>(y0), xb = qb<O>(x0);
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
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          acc[c] = fmaf(w00, v00[c], acc[c]);
          acc[c] = fmaf(w01, v01[c], acc[c]);
          acc[c] = fmaf(w10, v10[c], acc[c]);
          acc[c] = fmaf(w11, v11[c], acc[c]);
        }
      };
      fix(I0{});
      if constexpr (r < 2) {
        fix(I1{});
        fix(I2{});
        fix(I3{});
      }
    };
    fix_round(I0{});
    fix_round(I1{});
    fix_round(I2{});

    pack_words<DT, CPL>(acc, outw);
    out_off = cur.live ? (cur.pg * CG + sub * CPL) * io::kBytes : kOutOfRange;
    have_out = true;

    if (!more) break;
    item = next;
    cur = decode(item);
    buf ^= 1;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      off[r] = off_n[r];
      lg[r] = lg_n[r];
    }
  }
  if constexpr (NW == 4) {
    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(v4{outw[0], outw[1], outw[2], outw[3]}, rout, (int)out_off, 0, 0);
  } else {
    typedef uint32_t v2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(v2{outw[0], outw[1]}, rout, (int)out_off, 0, 0);
  }
}

namespace {

template <int DT, bool SM>
hipError_t launch_quad(const FwdParams &p, const QuadGeom &qg, hipStream_t s) {
  auto kern = dcn_fwd_quad_kernel<DT, SM>;
  const size_t lds = 2 * (size_t)qg.buf_bytes;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const uint32_t blocks = std::min<uint32_t>(qg.t.items, (uint32_t)cus);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kQuadThreads), lds, s, p, qg);
  return hipGetLastError();
}

}  // namespace

// 3x3 points whose two window buffers fit 160 KB of LDS; hipErrorNotSupported
// (nothing launched) otherwise.
hipError_t launch_forward_quad(int dtype, int softmax, const FwdParams &p, hipStream_t s) {
  if (p.KH != 3 || p.KW != 3) return hipErrorNotSupported;
  QuadGeom qg{};
  TileGeom &tg = qg.t;
  tg.span_h = (kQuadTile - 1) * p.SH + 2 * p.DH + 2 * kQuadHalo + 2;
  tg.span_w = (kQuadTile - 1) * p.SW + 2 * p.DW + 2 * kQuadHalo + 2;
  const int pixb = dtype == DCN_F32 ? quad_pixb<DCN_F32>() : quad_pixb<DCN_F16>();
  const int64_t win = (int64_t)tg.span_h * tg.span_w * pixb;
  const int64_t zero = (int64_t)tg.span_w * pixb + 2 * pixb;  // what a sample outside reads
  const int64_t ndma = (win + 1023) / 1024;                   // the last block may spill into the zero block
  int64_t buf = (win + zero + 1023) / 1024 * 1024;
  if (ndma * 1024 > buf) buf = ndma * 1024;
  if (2 * buf > 160 * 1024) return hipErrorNotSupported;
  qg.buf_bytes = (int32_t)buf;
  qg.ndma = (int32_t)ndma;
  const int tiles_y = (p.Ho + kQuadTile - 1) / kQuadTile;
  tg.tiles_x = (p.Wo + kQuadTile - 1) / kQuadTile;
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
    case DCN_F32: return softmax ? launch_quad<DCN_F32, true>(p, qg, s) : launch_quad<DCN_F32, false>(p, qg, s);
    case DCN_F16: return softmax ? launch_quad<DCN_F16, true>(p, qg, s) : launch_quad<DCN_F16, false>(p, qg, s);
    case DCN_BF16: return softmax ? launch_quad<DCN_BF16, true>(p, qg, s) : launch_quad<DCN_BF16, false>(p, qg, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dcn
