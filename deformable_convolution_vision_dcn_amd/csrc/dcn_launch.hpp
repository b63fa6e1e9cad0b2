// dcn_launch.hpp -- the library's internal interface between the C ABI
// (validation, chunking) and the kernels.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn.h"
#include "index_math.hpp"

namespace dcn {

constexpr int kGroupChannels = 16;  // channels per group with a kernel
constexpr int kMaxPoints = 64;      // sampling points per pixel-group, upper bound
constexpr int kBlock = 256;         // threads per block of every kernel

// One launch covers a chunk of whole images whose input stays below 2^31
// bytes, so every corner address fits a 32-bit buffer offset.
struct FwdParams {
  const void *input;   // chunk's first image
  const void *offset;
  const void *mask;
  void *output;
  uint32_t in_bytes;   // bytes of the chunk's input (buffer num_records)
  uint32_t off_bytes;  // bytes of the chunk's offset, mask and output tensors
  uint32_t mask_bytes; // (each below 2^31, like the input)
  uint32_t out_bytes;
  uint32_t pg_total;   // pixel-groups (n, ho, wo, g) in the chunk
  int32_t H, W, C, G, Ho, Wo;
  int32_t KH, KW, SH, SW, PH, PW, DH, DW;
  int32_t RC;          // 1: the centre point is not sampled (K = KH*KW - 1)
  float scale;
  FastDiv div_g, div_wo, div_ho;
};

struct BwdParams {
  FwdParams f;             // input, offset, mask and geometry as in the forward
  const void *grad_out;    // (chunk, Ho, Wo, C), the I/O dtype like every tensor
  void *grad_in;           // (chunk, H, W, C): the whole-map kernel writes it in the I/O dtype;
                           // the others add into it in fp32 (for 16-bit I/O the fp32
                           // accumulator), zeroed before the launch
  void *acc;               // whole-map kernel: fp32 (chunk, H, W, C) accumulator of items on
                           // fp32 atomics (grad_in itself for fp32 I/O); contents on entry unused
  void *grad_offset;       // (chunk, Ho, Wo, G, K, 2)
  void *grad_mask;         // (chunk, Ho, Wo, G, K)
};

// The forward fused with the linear steps around the core: offsets and mask
// generated from a guide feature, or an output projection after it.
struct FusedParams {
  FwdParams f;             // geometry, input, output; offset and mask when not generated
  uint32_t npix;           // output pixels of the chunk (N * Ho * Wo)
  int32_t gc;              // groups per chunk (set by the launcher)
  const void *guide;       // (chunk, Ho, Wo, cgd)
  uint32_t guide_bytes;
  int32_t cgd;             // guide channels, a multiple of 8
  const void *w_off;       // (G*K*2, cgd)
  const void *b_off;       // (G*K*2) or NULL
  const void *w_mask;      // (G*K, cgd)
  const void *b_mask;      // (G*K) or NULL
  uint32_t w_off_bytes, w_mask_bytes;
  const void *w_out;       // (C, C)
  const void *b_out;       // (C) or NULL
  uint32_t w_out_bytes;
};

// Geometry of the LDS-tiled forward: one block per (image, output tile,
// group); the input window of the tile (plus a halo of R pixels on every
// side for the learned offsets) is staged into LDS.
struct TileGeom {
  int32_t span_h, span_w;    // staged window, in input pixels
  int32_t tiles_x, tiles_per_img;
  uint32_t items;            // (image, tile, group) work items of the launch
  FastDiv div_g, div_tiles, div_tiles_x, div_span_w;
};

hipError_t launch_forward(int dtype, int softmax, const FwdParams &p, hipStream_t s);
hipError_t launch_forward_tiled(int dtype, int softmax, const FwdParams &p, hipStream_t s,
                                int groups_per_item);
hipError_t launch_forward_lane(int dtype, int softmax, const FwdParams &p, hipStream_t s);
hipError_t launch_forward_map(int dtype, int softmax, const FwdParams &p, hipStream_t s);
// The backward; `whole_map` (from backward_takes_map) selects the whole-map
// kernel, which writes grad_in in the I/O dtype without a prior clear.
hipError_t launch_backward(int dtype, int softmax, const BwdParams &p, bool whole_map, hipStream_t s);
// Whether the backward of this problem runs the whole-map kernel (read at
// every call: the DCN_MI355X_BWD_PATH override can turn it off).
bool backward_takes_map(const FwdParams &p);
bool backward_map_applies(const FwdParams &p);
hipError_t launch_backward_map(int dtype, int softmax, const BwdParams &p, hipStream_t s);
hipError_t launch_backward_tiled(int softmax, const BwdParams &p, hipStream_t s);
hipError_t launch_backward_quad(int dtype, int softmax, const BwdParams &p, hipStream_t s);
hipError_t launch_forward_generated(int dtype, int softmax, const FusedParams &p, hipStream_t s);
hipError_t launch_forward_projected(int dtype, int softmax, const FusedParams &p, hipStream_t s);
// Whether the fused kernel's LDS holds this problem (G groups of K points, C channels).
bool fused_fits(int G, int K, int C, bool proj);
hipError_t launch_zero(void *dst, uint64_t bytes, hipStream_t s);
// dst (16-bit dtype, count elements) = src (fp32) rounded; count % 8 == 0.
hipError_t launch_narrow(int dtype, const void *src, void *dst, uint64_t count, hipStream_t s);

}  // namespace dcn
