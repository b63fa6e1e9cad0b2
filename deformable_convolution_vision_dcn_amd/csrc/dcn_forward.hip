// dcn_forward.hip -- gfx950 forward kernel of the DCNv3/DCNv4 sampling core.
//
// Operation (wmrh.cn/news/61976, section 二 steps 2-4 and section 三; the
// unnormalised DCNv4 mask on pnsm.cn/news/2029644.html, section 2.2): for each
// output pixel, group and kernel point, move the regular grid position by
// offset_scale times the learned (x, y) offset, bilinearly sample the group's
// 16-channel slice of the NHWC map (zero outside), weight it by the point's
// modulation scalar (softmax over the points for DCNv3, raw for DCNv4) and sum.
//
// Design (gfx950): a gather-reduce, so VALU + vector memory, no MFMA.
//  * One block = 256 threads = BLOCK_PG consecutive pixel-groups (LANES lanes
//    per pixel-group, CPL = 16 / LANES channels per lane).  Consecutive
//    pixel-groups are the groups of consecutive pixels, so the block's offset
//    and mask rows are one contiguous span: it is staged once into LDS with
//    16-byte loads and read back per lane.
//  * The sampling location is split into floor and fraction of s*offset
//    before the integer grid index is added, so the fraction is exact for
//    power-of-two offset_scale at any map size.  The four bilinear weights
//    are computed once per point, with the modulation scalar folded in, and
//    shared by all channels of the lane: 4 FMAs per channel per point.
//  * Corner slices are read with raw buffer loads; a corner outside the map
//    gets a byte offset beyond the buffer's extent, which the hardware returns
//    as zero -- zero padding without a branch.
//  * Blocks are remapped so that each XCD owns a contiguous run of pixels and
//    the overlapping sampling windows of neighbouring pixels meet in its L2.
#include <stdlib.h>
#include <string.h>

#include "dcn_device.hpp"

namespace dcn {

template <int DT>
__device__ __forceinline__ float lds_get(const void *lds, uint32_t i) {
  if constexpr (DT == DCN_F32) {
    return static_cast<const float *>(lds)[i];
  } else if constexpr (DT == DCN_F16) {
    return (float)static_cast<const _Float16 *>(lds)[i];
  } else {
    return __uint_as_float((uint32_t) static_cast<const uint16_t *>(lds)[i] << 16);
  }
}

// KH_ = KW_ = 0 selects run-time kernel extents.
template <int DT, int LANES, int KH_, int KW_, bool SOFTMAX>
__global__ void __launch_bounds__(kBlock) dcn_fwd_kernel(FwdParams p) {
  using io = Io<DT>;
  constexpr int CG = kGroupChannels;
  constexpr int CPL = CG / LANES;                 // channels per lane
  constexpr int NW = CPL * io::kBytes / 4;        // 32-bit words per lane per corner
  constexpr int BLOCK_PG = kBlock / LANES;
  constexpr bool FIXED = KH_ > 0;
  const int KH = FIXED ? KH_ : p.KH;
  const int KW = FIXED ? KW_ : p.KW;
  const int K = FIXED ? KH_ * KW_ : KH * KW - p.RC;  // fixed extents never drop the centre

  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char *lds_off = lds;
  unsigned char *lds_mask = lds + (uint32_t)BLOCK_PG * K * 2 * io::kBytes;

  const uint32_t blk = xcd_block(blockIdx.x, gridDim.x);
  const uint32_t pg0 = blk * BLOCK_PG;
  const uint32_t npg = min((uint32_t)BLOCK_PG, p.pg_total - pg0);
  stage_to_lds(lds_off, static_cast<const unsigned char *>(p.offset) + (uint64_t)pg0 * K * 2 * io::kBytes,
               npg * K * 2 * io::kBytes);
  stage_to_lds(lds_mask, static_cast<const unsigned char *>(p.mask) + (uint64_t)pg0 * K * io::kBytes,
               npg * K * io::kBytes);
  __syncthreads();

  const uint32_t lp = threadIdx.x / LANES;
  const uint32_t sub = threadIdx.x % LANES;
  if (lp >= npg) return;
  const uint32_t pg = pg0 + lp;

  // (n, ho, wo, g) of this pixel-group; pg = ((n*Ho + ho)*Wo + wo)*G + g.
  const uint32_t pix = fast_div(pg, p.div_g);
  const uint32_t g = pg - pix * (uint32_t)p.G;
  const uint32_t t = fast_div(pix, p.div_wo);
  const uint32_t wo = pix - t * (uint32_t)p.Wo;
  const uint32_t n = fast_div(t, p.div_ho);
  const uint32_t ho = t - n * (uint32_t)p.Ho;

  // Modulation scalars: softmax over the K points (max-subtracted) or raw.
  const uint32_t mrow = lp * K;
  float mx = 0.f, inv = 1.f;
  float mfix[FIXED ? KH_ * KW_ : 1];
  if constexpr (SOFTMAX) {
    mx = -INFINITY;
    for (int k = 0; k < K; ++k) mx = fmaxf(mx, lds_get<DT>(lds_mask, mrow + k));
    float sum = 0.f;
    for (int k = 0; k < K; ++k) {
      const float e = __expf(lds_get<DT>(lds_mask, mrow + k) - mx);
      if constexpr (FIXED) mfix[k] = e;
      sum += e;
    }
    inv = __builtin_amdgcn_rcpf(sum);
  }

  const uint32_t pix_bytes = (uint32_t)p.C * io::kBytes;
  const uint32_t row_bytes = (uint32_t)p.W * pix_bytes;
  const uint32_t base = n * (uint32_t)p.H * row_bytes + (g * CG + sub * CPL) * io::kBytes;
  const __amdgpu_buffer_rsrc_t rin = make_rsrc(p.input, p.in_bytes);
  const int by = (int)ho * p.SH - p.PH;
  const int bx = (int)wo * p.SW - p.PW;
  const float s = p.scale;

  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  bool nan_loc = false;

  // Point k at grid position (ii, jj): location, weights, four corner
  // gathers, FMAs.
  auto point = [&](const int ii, const int jj, const int k) {
    const uint32_t o = (mrow + k) * 2;
    const float dx = s * lds_get<DT>(lds_off, o);
    const float dy = s * lds_get<DT>(lds_off, o + 1);
    nan_loc |= (dx != dx) | (dy != dy);
    // Clamp first (|s*offset| >= 2^24 is far outside any map, and an infinite
    // offset must not turn the fraction into Inf - Inf), then split into an
    // integer part and an exact fraction in [0, 1).
    const float cx = __builtin_amdgcn_fmed3f(dx, -16777216.f, 16777216.f);
    const float cy = __builtin_amdgcn_fmed3f(dy, -16777216.f, 16777216.f);
    const float fx = floorf(cx), fy = floorf(cy);
    const float lx = cx - fx, ly = cy - fy;
    const int x0 = bx + jj * p.DW + (int)fx;
    const int y0 = by + ii * p.DH + (int)fy;

    float mk;
    if constexpr (!SOFTMAX) {
      mk = lds_get<DT>(lds_mask, mrow + k);
    } else if constexpr (FIXED) {
      mk = mfix[k] * inv;
    } else {
      mk = __expf(lds_get<DT>(lds_mask, mrow + k) - mx) * inv;
    }
    const float wy0 = (1.f - ly) * mk, wy1 = ly * mk;
    const float w00 = wy0 * (1.f - lx), w01 = wy0 * lx;
    const float w10 = wy1 * (1.f - lx), w11 = wy1 * lx;

    const bool vy0 = (uint32_t)y0 < (uint32_t)p.H, vy1 = (uint32_t)(y0 + 1) < (uint32_t)p.H;
    const bool vx0 = (uint32_t)x0 < (uint32_t)p.W, vx1 = (uint32_t)(x0 + 1) < (uint32_t)p.W;
    const uint32_t a00 = base + (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_bytes;
    const uint32_t a01 = a00 + pix_bytes, a10 = a00 + row_bytes, a11 = a10 + pix_bytes;

    uint32_t q00[NW], q01[NW], q10[NW], q11[NW];
    buffer_load_words<NW>(rin, (vy0 && vx0) ? a00 : kOutOfRange, q00);
    buffer_load_words<NW>(rin, (vy0 && vx1) ? a01 : kOutOfRange, q01);
    buffer_load_words<NW>(rin, (vy1 && vx0) ? a10 : kOutOfRange, q10);
    buffer_load_words<NW>(rin, (vy1 && vx1) ? a11 : kOutOfRange, q11);
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
  if constexpr (FIXED) {
#pragma unroll
    for (int ii = 0; ii < KH_; ++ii)
#pragma unroll
      for (int jj = 0; jj < KW_; ++jj) point(ii, jj, ii * KW_ + jj);
  } else {
    // Row-major over the grid; with RC the centre is skipped and the points
    // after it take the next indices.
    const int centre = p.RC ? (KH / 2) * KW + KW / 2 : -1;
    for (int q = 0, k = 0; q < KH * KW; ++q) {
      if (q == centre) continue;
      const int ii = q / KW;
      point(ii, q - ii * KW, k++);
    }
  }

  if (nan_loc) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = __builtin_nanf("");
  }
  uint32_t out[NW];
  pack_words<DT, CPL>(acc, out);
  store_words<NW>(static_cast<unsigned char *>(p.output) +
                      ((uint64_t)pg * CG + sub * CPL) * io::kBytes,
                  out);
}

namespace {

template <int DT, int LANES, int KH, int KW, bool SM>
hipError_t launch_one(const FwdParams &p, hipStream_t s) {
  constexpr int BLOCK_PG = kBlock / LANES;
  const int K = p.KH * p.KW - p.RC;
  const size_t lds = (size_t)BLOCK_PG * K * 3 * Io<DT>::kBytes;
  const uint32_t blocks = (p.pg_total + BLOCK_PG - 1) / BLOCK_PG;
  hipLaunchKernelGGL((dcn_fwd_kernel<DT, LANES, KH, KW, SM>), dim3(blocks), dim3(kBlock), lds, s, p);
  return hipGetLastError();
}

// Lanes per pixel-group of the untiled kernel: four (4 fp32 channels per lane)
// for fp32, two (8 channels, one 16-byte load per corner) for 16-bit I/O.
template <int DT>
hipError_t launch_dt(int softmax, const FwdParams &p, hipStream_t s) {
  constexpr int LANES = DT == DCN_F32 ? 4 : 2;
  const bool k33 = p.KH == 3 && p.KW == 3 && !p.RC;
  if (k33) {
    return softmax ? launch_one<DT, LANES, 3, 3, true>(p, s) : launch_one<DT, LANES, 3, 3, false>(p, s);
  }
  return softmax ? launch_one<DT, LANES, 0, 0, true>(p, s) : launch_one<DT, LANES, 0, 0, false>(p, s);
}

// Forward path override for tests and measurements: DCN_MI355X_FWD_PATH =
// "generic", "tiled" (one group per work item), "pair" (two groups per work
// item), "lane" or "map" tries that kernel first (and falls back to the
// generic kernel where it does not apply).  Read at every call.
enum class Path { kAuto, kGeneric, kTiled, kPair, kLane, kMap };

Path path_override() {
  const char *e = getenv("DCN_MI355X_FWD_PATH");
  if (!e) return Path::kAuto;
  if (!strcmp(e, "generic")) return Path::kGeneric;
  if (!strcmp(e, "tiled")) return Path::kTiled;
  if (!strcmp(e, "pair")) return Path::kPair;
  if (!strcmp(e, "lane")) return Path::kLane;
  if (!strcmp(e, "map")) return Path::kMap;
  return Path::kAuto;
}

}  // namespace

// Kernel choice for 3x3 points: an output map smaller than one 16x16 tile
// (or one that tiles would leave over half empty) whose bordered window, of
// one or more groups, fits in LDS runs the whole-map kernel (every lane
// busy, several groups per item, no halo re-reads, no global fix-ups).  Other maps that
// fit a tile window: fp32 runs the quad tiled kernel (a quad of lanes per
// pixel-group; two groups per work item where the group count is even; also
// at stride 2 and dilation 2, and without the kernel's centre), 16-bit I/O
// the lane-per-pixel-group kernel at stride and dilation 1 (one, two or four
// groups per work item), which needs a quarter of the address and weight
// arithmetic and wins once a pixel's 16 channels are only 32 bytes, and the
// quad tiled kernel at other strides and dilations.  5x5 points at stride
// and dilation 1 run the lane kernel in every dtype.  Everything else runs
// the untiled kernel.
// Whether the whole-map kernel is the first choice: the output map is
// smaller than one 16x16 tile, or tiles would leave over half of their
// pixel slots empty.  (At 24x24, 56 % full, the tiled lane kernel is still
// faster: with one group per item the whole-map kernel's rows are scattered.)
static bool prefer_map(const FwdParams &p) {
  const int64_t ty = (p.Ho + 15) / 16, tx = (p.Wo + 15) / 16;
  const int64_t area = (int64_t)p.Ho * p.Wo;
  return area < 256 || 2 * area < ty * tx * 256;
}

hipError_t launch_forward(int dtype, int softmax, const FwdParams &p, hipStream_t s) {
  const Path forced = path_override();
  if (forced == Path::kMap || (forced == Path::kAuto && prefer_map(p))) {
    const hipError_t m = launch_forward_map(dtype, softmax, p, s);
    if (m != hipErrorNotSupported) return m;
  }
  const bool lane_first = forced == Path::kLane || (forced == Path::kAuto && dtype != DCN_F32);
  if (forced != Path::kGeneric && forced != Path::kMap) {
    if (lane_first) {
      const hipError_t l = launch_forward_lane(dtype, softmax, p, s);
      if (l != hipErrorNotSupported) return l;
    }
    if (forced != Path::kLane) {
      const int gpi = forced == Path::kTiled ? 1 : (forced == Path::kPair ? 2 : 0);
      const hipError_t t = launch_forward_tiled(dtype, softmax, p, s, gpi);
      if (t != hipErrorNotSupported) return t;
    }
    if (!lane_first && forced == Path::kAuto) {  // fp32 problems whose window the tiled kernels refuse
      const hipError_t l = launch_forward_lane(dtype, softmax, p, s);
      if (l != hipErrorNotSupported) return l;
    }
  }
  switch (dtype) {
    case DCN_F32: return launch_dt<DCN_F32>(softmax, p, s);
    case DCN_F16: return launch_dt<DCN_F16>(softmax, p, s);
    case DCN_BF16: return launch_dt<DCN_BF16>(softmax, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dcn
