// dcn_fwd_tile.hip -- LDS-tiled gfx950 forward kernel of the DCN core for
// 3x3 kernel points (the InternImage configuration; wmrh.cn/news/61976,
// section 二 steps 2-4 and section 三).
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
// address of the kernel points k = sub, sub+4, sub+8; DPP quad broadcasts
// hand them to the other three lanes, so no lane repeats another's address
// math.  Each lane then reads its 16-byte chunk of the four corners and does
// 4 FMAs per channel per point.  The softmax over the nine logits is a quad
// reduction (max, then sum of exponentials).
#include <type_traits>

#include "dcn_device.hpp"

namespace dcn {

namespace {

template <int O>
__device__ __forceinline__ int qbcast(int v) {
  constexpr int ctrl = O | (O << 2) | (O << 4) | (O << 6);  // quad_perm [O,O,O,O]
  return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, false);
}
template <int O>
__device__ __forceinline__ float qbcast(float v) {
  return __int_as_float(qbcast<O>(__float_as_int(v)));
}

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return v;
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  return v;
}

template <int NW>
__device__ __forceinline__ void lds_store(unsigned char *dst, const uint32_t (&w)[NW]) {
  if constexpr (NW == 4) {
    *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
  }
}
template <int NW>
__device__ __forceinline__ void lds_load(const unsigned char *src, uint32_t (&w)[NW]) {
  if constexpr (NW == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(src);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2 *>(src);
    w[0] = v.x; w[1] = v.y;
  }
}

// (x, y) offset pair of element pair index e, widened to fp32.
template <int DT>
__device__ __forceinline__ float2 load_pair(const void *base, uint32_t e) {
  if constexpr (DT == DCN_F32) {
    return static_cast<const float2 *>(base)[e];
  } else {
    const uint32_t w = static_cast<const uint32_t *>(base)[e];
    return make_float2(Io<DT>::lo(w), Io<DT>::hi(w));
  }
}
template <int DT>
__device__ __forceinline__ float load_one(const void *base, uint32_t e) {
  if constexpr (DT == DCN_F32) {
    return static_cast<const float *>(base)[e];
  } else if constexpr (DT == DCN_F16) {
    return (float)static_cast<const _Float16 *>(base)[e];
  } else {
    return __uint_as_float((uint32_t) static_cast<const uint16_t *>(base)[e] << 16);
  }
}

}  // namespace

#ifndef DCN_TILE_WAVES
#define DCN_TILE_WAVES 4  // waves per SIMD the register budget must allow
#endif
#ifndef DCN_PIXB_F32
#define DCN_PIXB_F32 80   // LDS bytes per staged fp32 pixel slice (64 + pad)
#endif
#ifndef DCN_PIXB_16
#define DCN_PIXB_16 40    // LDS bytes per staged 16-bit pixel slice (32 + pad)
#endif

template <int DT>
constexpr int tile_pixel_stride() { return DT == DCN_F32 ? DCN_PIXB_F32 : DCN_PIXB_16; }

template <int DT, bool SOFTMAX, int TH, int TW, int R>
__global__ void __launch_bounds__(512, DCN_TILE_WAVES) dcn_fwd_tile_kernel(FwdParams p, TileGeom tg) {
  using io = Io<DT>;
  constexpr int CG = kGroupChannels;
  constexpr int CPL = 4;                           // channels per lane
  constexpr int NW = CPL * io::kBytes / 4;         // words per lane per corner
  constexpr int LANE_BYTES = CPL * io::kBytes;
  constexpr int PIXB = tile_pixel_stride<DT>();
  constexpr int QUADS = 512 / 4;
  constexpr int PASSES = TH * TW / QUADS;
  constexpr int K = 9;
  static_assert((TH * TW) % QUADS == 0, "tile must be a multiple of the quad count");
  static_assert(PIXB % LANE_BYTES == 0 && PIXB % 8 == 0 && PIXB >= 4 * LANE_BYTES, "pixel stride");

  extern __shared__ __align__(16) unsigned char tile[];

  // Logical block -> (n, tile, g); g varies fastest so the blocks that share
  // an input window's cache lines (neighbouring groups) run together.
  const uint32_t b = xcd_block(blockIdx.x, gridDim.x);
  const uint32_t t = fast_div(b, tg.div_g);
  const uint32_t g = b - t * (uint32_t)p.G;
  const uint32_t n = fast_div(t, tg.div_tiles);
  const uint32_t tile_id = t - n * (uint32_t)tg.tiles_per_img;
  const uint32_t tyi = fast_div(tile_id, tg.div_tiles_x);
  const uint32_t txi = tile_id - tyi * (uint32_t)tg.tiles_x;
  const int r0 = (int)tyi * TH, c0 = (int)txi * TW;
  const int Y0 = r0 * p.SH - p.PH - R;   // window origin in input coordinates
  const int X0 = c0 * p.SW - p.PW - R;

  const uint32_t quad = threadIdx.x >> 2, sub = threadIdx.x & 3;
  const uint32_t pix_bytes = (uint32_t)p.C * io::kBytes;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const uint32_t chan = (g * CG + sub * CPL) * io::kBytes;
  const uint32_t img = n * (uint32_t)p.H * row_bytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);

  // ---- own points' offsets and logits of every pass, requested before the
  // window so that both latencies overlap.  Quad `quad` of pass `ps` owns
  // output pixel pp = ps*QUADS + quad of the tile; lane `sub` owns the
  // points k = sub + 4r.
  float2 off[PASSES][3];
  float lg[PASSES][3];
  uint32_t pgs[PASSES];
  bool live[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int pp = ps * QUADS + (int)quad;
    const int ho = r0 + pp / TW, wo = c0 + pp % TW;
    live[ps] = ho < p.Ho && wo < p.Wo;
    pgs[ps] = (((n * (uint32_t)p.Ho + ho) * (uint32_t)p.Wo + wo) * (uint32_t)p.G) + g;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int k = (int)sub + 4 * r;
      if (live[ps] && k < K) {
        off[ps][r] = load_pair<DT>(p.offset, pgs[ps] * K + k);
        lg[ps][r] = load_one<DT>(p.mask, pgs[ps] * K + k);
      } else {
        off[ps][r] = make_float2(0.f, 0.f);
        lg[ps][r] = SOFTMAX ? -INFINITY : 0.f;
      }
    }
  }

  // ---- stage the window: one quad per pixel, 4 pixels in flight per lane
  const int span = tg.span_h * tg.span_w;
  const int row_lds = tg.span_w * PIXB;
  for (int base = (int)quad; base < span; base += QUADS * 4) {
    uint32_t w[4][NW];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + u * QUADS;
      uint32_t offb = kOutOfRange;
      if (idx < span) {
        const int sy = (int)fast_div((uint32_t)idx, tg.div_span_w);
        const int sx = idx - sy * tg.span_w;
        const int gy = Y0 + sy, gx = X0 + sx;
        if ((uint32_t)gy < (uint32_t)p.H && (uint32_t)gx < (uint32_t)p.W)
          offb = img + (uint32_t)gy * row_bytes + (uint32_t)gx * pix_bytes + chan;
      }
      buffer_load_words<NW>(rin, offb, w[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = base + u * QUADS;
      if (idx < span) lds_store<NW>(tile + idx * PIXB + sub * LANE_BYTES, w[u]);
    }
  }
  // A zero block after the window: samples served from global memory (and
  // NaN locations) read their main-path corners here, contributing w * 0.
  const int zero_base = span * PIXB;
  for (int z = (int)threadIdx.x * 8; z < row_lds + 2 * PIXB; z += 512 * 8)
    *reinterpret_cast<uint2 *>(tile + zero_base + z) = make_uint2(0, 0);
  __syncthreads();

  const int lim_y = tg.span_h - 2, lim_x = tg.span_w - 2;
  const float s = p.scale;

  auto pass = [&](auto ps_tag) {
    constexpr int ps = decltype(ps_tag)::value;
    if (!live[ps]) return;  // whole quad leaves together
    const int pp = ps * QUADS + (int)quad;
    const int ho = r0 + pp / TW, wo = c0 + pp % TW;

    float m[3];
    if constexpr (SOFTMAX) {
      const float mx = quad_max(fmaxf(fmaxf(lg[ps][0], lg[ps][1]), lg[ps][2]));
      float e[3], sum = 0.f;
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        e[r] = ((int)sub + 4 * r < K) ? __expf(lg[ps][r] - mx) : 0.f;
        sum += e[r];
      }
      const float inv = __builtin_amdgcn_rcpf(quad_sum(sum));
#pragma unroll
      for (int r = 0; r < 3; ++r) m[r] = e[r] * inv;
    } else {
#pragma unroll
      for (int r = 0; r < 3; ++r) m[r] = lg[ps][r];
    }

    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;

    // Round r: every lane prepares its own point k = sub + 4r (location,
    // weights with the modulation folded in, window address), then the quad
    // consumes the round's points one owner at a time.  The per-round inputs
    // rotate through scalars (no run-time indexed arrays, so no scratch).
    float2 o2 = off[ps][0], o2n = off[ps][1], o2nn = off[ps][2];
    float mk = m[0], mkn = m[1], mknn = m[2];
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
      const int x0 = wo * p.SW - p.PW + j * p.DW + (int)fx;
      const int y0 = ho * p.SH - p.PH + i * p.DH + (int)fy;
      const float wy0 = (1.f - ly) * mk, wy1 = ly * mk;
      const float nanv = __builtin_nanf("");
      const float W0 = nan_loc ? nanv : wy0 * (1.f - lx);
      const float W1 = nan_loc ? nanv : wy0 * lx;
      const float W2 = nan_loc ? nanv : wy1 * (1.f - lx);
      const float W3 = nan_loc ? nanv : wy1 * lx;
      const int ty = y0 - Y0, tx = x0 - X0;
      const bool inside = !nan_loc && (uint32_t)ty <= (uint32_t)lim_y && (uint32_t)tx <= (uint32_t)lim_x;
      const int A = inside ? ty * row_lds + tx * PIXB : zero_base;
      // outside the window but touching the map: needs the global fix-up
      const bool fb = !inside && !nan_loc && (uint32_t)(y0 + 1) <= (uint32_t)p.H &&
                      (uint32_t)(x0 + 1) <= (uint32_t)p.W;

      // Main path, no branches: gather the round's corners from LDS.
      auto point = [&](auto o_tag) {
        constexpr int O = decltype(o_tag)::value;
        const int a = qbcast<O>(A);
        const float w00 = qbcast<O>(W0), w01 = qbcast<O>(W1);
        const float w10 = qbcast<O>(W2), w11 = qbcast<O>(W3);
        uint32_t q00[NW], q01[NW], q10[NW], q11[NW];
        const unsigned char *src = tile + a + sub * LANE_BYTES;
        lds_load<NW>(src, q00);
        lds_load<NW>(src + PIXB, q01);
        lds_load<NW>(src + row_lds, q10);
        lds_load<NW>(src + row_lds + PIXB, q11);
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
      // Fix-up for points whose corners left the window: global gathers,
      // the buffer range check reading 0 for corners outside the map.
      auto fixup = [&](auto o_tag) {
        constexpr int O = decltype(o_tag)::value;
        if (!qbcast<O>((int)fb)) return;
        const float w00 = qbcast<O>(W0), w01 = qbcast<O>(W1);
        const float w10 = qbcast<O>(W2), w11 = qbcast<O>(W3);
        const int yb = qbcast<O>(y0), xb = qbcast<O>(x0);
        const bool vy0 = (uint32_t)yb < (uint32_t)p.H, vy1 = (uint32_t)(yb + 1) < (uint32_t)p.H;
        const bool vx0 = (uint32_t)xb < (uint32_t)p.W, vx1 = (uint32_t)(xb + 1) < (uint32_t)p.W;
        const uint32_t a00 = img + (uint32_t)yb * row_bytes + (uint32_t)xb * pix_bytes + chan;
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
      if (__builtin_amdgcn_ballot_w64(fb) != 0) {  // rare: some quad of the wave left its window
        fixup(I0{});
        if (r < 2) {
          fixup(I1{});
          fixup(I2{});
          fixup(I3{});
        }
      }
      o2 = o2n;
      o2n = o2nn;
      mk = mkn;
      mkn = mknn;
    }

    uint32_t outw[NW];
    pack_words<DT, CPL>(acc, outw);
    store_words<NW>(static_cast<unsigned char *>(p.output) + ((uint64_t)pgs[ps] * CG + sub * CPL) * io::kBytes,
                    outw);
  };
  static_assert(PASSES == 2, "the pass sequence below assumes two passes");
  pass(std::integral_constant<int, 0>{});
  pass(std::integral_constant<int, 1>{});
}

namespace {

constexpr int kTileH = 16, kTileW = 16, kHalo = 6;
constexpr int kTileLdsLimit = 80 * 1024;  // two blocks per CU

size_t tile_lds_bytes(const TileGeom &tg, int pixb) {
  return ((size_t)tg.span_h * tg.span_w + tg.span_w + 2) * pixb;  // window + zero block
}

template <int DT, bool SM>
hipError_t launch_tile(const FwdParams &p, const TileGeom &tg, uint32_t blocks, hipStream_t s) {
  auto kern = dcn_fwd_tile_kernel<DT, SM, kTileH, kTileW, kHalo>;
  const size_t lds = tile_lds_bytes(tg, tile_pixel_stride<DT>());
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, kTileLdsLimit);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(512), lds, s, p, tg);
  return hipGetLastError();
}

}  // namespace

// Returns hipErrorNotSupported (nothing launched) when the problem is not a
// 3x3 one or its window does not fit the LDS budget.
hipError_t launch_forward_tiled(int dtype, int softmax, const FwdParams &p, hipStream_t s) {
  if (p.KH != 3 || p.KW != 3) return hipErrorNotSupported;
  TileGeom tg{};
  tg.span_h = (kTileH - 1) * p.SH + 2 * p.DH + 2 * kHalo + 2;
  tg.span_w = (kTileW - 1) * p.SW + 2 * p.DW + 2 * kHalo + 2;
  const int pixb = dtype == DCN_F32 ? tile_pixel_stride<DCN_F32>() : tile_pixel_stride<DCN_F16>();
  if (tile_lds_bytes(tg, pixb) > (size_t)kTileLdsLimit) return hipErrorNotSupported;
  const int tiles_y = (p.Ho + kTileH - 1) / kTileH;
  tg.tiles_x = (p.Wo + kTileW - 1) / kTileW;
  tg.tiles_per_img = tiles_y * tg.tiles_x;
  const int64_t imgs = p.pg_total / ((int64_t)p.Ho * p.Wo * p.G);
  const int64_t blocks = imgs * tg.tiles_per_img * p.G;
  if (blocks <= 0 || blocks >= (int64_t(1) << 31)) return hipErrorNotSupported;
  tg.div_g = make_fast_div((uint32_t)p.G);
  tg.div_tiles = make_fast_div((uint32_t)tg.tiles_per_img);
  tg.div_tiles_x = make_fast_div((uint32_t)tg.tiles_x);
  tg.div_span_w = make_fast_div((uint32_t)tg.span_w);
  const uint32_t nb = (uint32_t)blocks;
  switch (dtype) {
    case DCN_F32: return softmax ? launch_tile<DCN_F32, true>(p, tg, nb, s) : launch_tile<DCN_F32, false>(p, tg, nb, s);
    case DCN_F16: return softmax ? launch_tile<DCN_F16, true>(p, tg, nb, s) : launch_tile<DCN_F16, false>(p, tg, nb, s);
    case DCN_BF16: return softmax ? launch_tile<DCN_BF16, true>(p, tg, nb, s) : launch_tile<DCN_BF16, false>(p, tg, nb, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dcn
