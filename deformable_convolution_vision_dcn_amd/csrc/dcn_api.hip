// dcn_api.hip -- the C ABI declared in include/dcn.h: problem validation,
// splitting a batch into launchable chunks of images, and the launches.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "dcn_launch.hpp"

// The fp32 grad_input accumulator of dcn_backward_noalloc's 16-bit chunks:
// device memory the library owns, one copy per GPU, held until the process
// ends.  Host code never passes this name to a kernel (on the host it is a
// stand-in, not a device address): it uses the address that
// hipGetSymbolAddress reports for the current device.
constexpr uint64_t kScratchBytes = uint64_t(DCN_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_hip_message[256] = "HIP error";

constexpr int64_t kMaxBytes31 = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxExtent = int64_t(1) << 24;

int64_t out_extent(int64_t in, int64_t k, int64_t stride, int64_t pad, int64_t dil) {
  const int64_t span = in + 2 * pad - dil * (k - 1) - 1;
  return span < 0 ? 0 : span / stride + 1;
}

int elem_bytes(int32_t dtype) { return dtype == DCN_F32 ? 4 : 2; }

// Sampling points per pixel-group: the kernel grid, less its centre with
// remove_center.
int64_t npoints(const dcn_problem *p) { return (int64_t)p->kernel_h * p->kernel_w - p->remove_center; }

// Every check of dcn_check, in a fixed order; fills ho/wo on success.
int validate(const dcn_problem *p, int64_t *ho_out, int64_t *wo_out) {
  if (!p) return DCN_ERR_NULL;
  if (p->struct_size != sizeof(dcn_problem)) return DCN_ERR_ABI;
  if (p->n < 0 || p->h <= 0 || p->w <= 0 || p->c <= 0 || p->groups <= 0) return DCN_ERR_SHAPE;
  if (p->c % p->groups != 0) return DCN_ERR_SHAPE;
  if (p->kernel_h <= 0 || p->kernel_w <= 0 || p->stride_h <= 0 || p->stride_w <= 0 ||
      p->dilation_h <= 0 || p->dilation_w <= 0 || p->pad_h < 0 || p->pad_w < 0)
    return DCN_ERR_SHAPE;
  if (p->softmax != 0 && p->softmax != 1) return DCN_ERR_ARG;
  if (p->remove_center != 0 && p->remove_center != 1) return DCN_ERR_ARG;
  if (p->remove_center && (p->kernel_h % 2 == 0 || p->kernel_w % 2 == 0)) return DCN_ERR_ARG;
  if (npoints(p) < 1) return DCN_ERR_SHAPE;
  if (!isfinite(p->offset_scale)) return DCN_ERR_ARG;
  if (p->h > kMaxExtent || p->w > kMaxExtent || p->pad_h > kMaxExtent || p->pad_w > kMaxExtent ||
      (int64_t)p->dilation_h * p->kernel_h > kMaxExtent ||
      (int64_t)p->dilation_w * p->kernel_w > kMaxExtent)
    return DCN_ERR_TOO_LARGE;
  const int64_t ho = out_extent(p->h, p->kernel_h, p->stride_h, p->pad_h, p->dilation_h);
  const int64_t wo = out_extent(p->w, p->kernel_w, p->stride_w, p->pad_w, p->dilation_w);
  if (ho < 1 || wo < 1) return DCN_ERR_SHAPE;
  if (p->dtype != DCN_F32 && p->dtype != DCN_F16 && p->dtype != DCN_BF16) return DCN_ERR_UNSUPPORTED;
  if (p->c / p->groups != dcn::kGroupChannels) return DCN_ERR_UNSUPPORTED;
  if (npoints(p) > dcn::kMaxPoints) return DCN_ERR_UNSUPPORTED;
  const int64_t img_bytes = (int64_t)p->h * p->w * p->c * elem_bytes(p->dtype);
  const int64_t img_out_bytes = ho * wo * p->c * elem_bytes(p->dtype);
  const int64_t img_off_bytes = ho * wo * p->groups * npoints(p) * 2 * elem_bytes(p->dtype);
  if (img_bytes > kMaxBytes31 || img_out_bytes > kMaxBytes31 || img_off_bytes > kMaxBytes31)
    return DCN_ERR_TOO_LARGE;
  if (ho_out) *ho_out = ho;
  if (wo_out) *wo_out = wo;
  return DCN_OK;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
// NULL or aligned to one element of `eb` bytes
bool aligned_elem(const void *ptr, int eb) { return (reinterpret_cast<uintptr_t>(ptr) & (uintptr_t)(eb - 1)) == 0; }

int hip_fail(hipError_t e) {
  snprintf(g_hip_message, sizeof(g_hip_message), "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return DCN_ERR_HIP;
}

// Geometry shared by every chunk of one call; the caller fills the pointers.
dcn::FwdParams geometry(const dcn_problem *p, int64_t ho, int64_t wo) {
  dcn::FwdParams f{};
  f.H = p->h;
  f.W = p->w;
  f.C = p->c;
  f.G = p->groups;
  f.Ho = (int32_t)ho;
  f.Wo = (int32_t)wo;
  f.KH = p->kernel_h;
  f.KW = p->kernel_w;
  f.SH = p->stride_h;
  f.SW = p->stride_w;
  f.PH = p->pad_h;
  f.PW = p->pad_w;
  f.DH = p->dilation_h;
  f.DW = p->dilation_w;
  f.RC = p->remove_center;
  f.scale = p->offset_scale;
  f.div_g = dcn::make_fast_div((uint32_t)p->groups);
  f.div_wo = dcn::make_fast_div((uint32_t)wo);
  f.div_ho = dcn::make_fast_div((uint32_t)ho);
  return f;
}

// Images per launch: every chunk keeps its input, output and offset tensors
// (the mask is half the offsets) below 2^31 bytes, the reach of the kernels'
// 32-bit buffer offsets (pixel-group indices then stay below 2^31 / 16 as
// well).
int64_t images_per_chunk(const dcn_problem *p, int64_t ho, int64_t wo) {
  const int64_t img_bytes = (int64_t)p->h * p->w * p->c * elem_bytes(p->dtype);
  const int64_t img_out_bytes = ho * wo * p->c * elem_bytes(p->dtype);
  const int64_t img_off_bytes = ho * wo * p->groups * npoints(p) * 2 * elem_bytes(p->dtype);
  int64_t per = kMaxBytes31 / img_bytes;
  const int64_t per2 = kMaxBytes31 / img_out_bytes;
  const int64_t per3 = kMaxBytes31 / img_off_bytes;
  if (per2 < per) per = per2;
  if (per3 < per) per = per3;
  return per < 1 ? 1 : per;
}

// The backward's extra check: for 16-bit I/O, one image's fp32 grad_input
// accumulator below 2^31 bytes.
int validate_backward(const dcn_problem *p, int64_t *ho, int64_t *wo) {
  const int st = validate(p, ho, wo);
  if (st != DCN_OK) return st;
  if (p->dtype == DCN_F32) return DCN_OK;
  if ((int64_t)p->h * p->w * p->c * 4 > kMaxBytes31) return DCN_ERR_TOO_LARGE;
  return DCN_OK;
}

// Images per backward launch: as for the forward, and for 16-bit I/O also
// the fp32 accumulator of the chunk's grad_input below 2^31 bytes.
int64_t images_per_chunk_bwd(const dcn_problem *p, int64_t ho, int64_t wo) {
  int64_t per = images_per_chunk(p, ho, wo);
  if (p->dtype != DCN_F32) {
    const int64_t per32 = kMaxBytes31 / ((int64_t)p->h * p->w * p->c * 4);
    if (per32 < per) per = per32;
  }
  return per < 1 ? 1 : per;
}

// fp32 accumulator bytes of the largest chunk (0 for fp32 I/O or N == 0).
uint64_t workspace_bytes_bwd(const dcn_problem *p, int64_t ho, int64_t wo) {
  if (p->dtype == DCN_F32 || p->n == 0) return 0;
  int64_t per = images_per_chunk_bwd(p, ho, wo);
  if (p->n < per) per = p->n;
  return (uint64_t)(per * p->h * p->w * p->c * 4);
}

// The enqueue stage of both backward entry points, after their checks:
// pointers are checked here, then the chunks of `per` images are launched.
// For 16-bit I/O `ws` is the fp32 accumulator of one chunk (per*H*W*C*4
// bytes at least).
int run_backward(const dcn_problem *p, int64_t ho, int64_t wo, const void *input, const void *offset,
                 const void *mask, const void *grad_output, void *grad_input, void *grad_offset, void *grad_mask,
                 void *ws, int64_t per, void *hip_stream) {
  const bool wide = p->dtype == DCN_F32;  // grad_input accumulates in place
  if (!input || !offset || !mask || !grad_output || !grad_input || !grad_offset || !grad_mask) return DCN_ERR_NULL;
  if (!aligned16(input) || !aligned16(offset) || !aligned16(mask) || !aligned16(grad_output) ||
      !aligned16(grad_input) || !aligned16(grad_offset) || !aligned16(grad_mask))
    return DCN_ERR_ALIGN;

  const int64_t K = npoints(p);
  const int64_t eb = elem_bytes(p->dtype);
  const int64_t img_elems = (int64_t)p->h * p->w * p->c;
  const int64_t img_in = img_elems * eb;
  const int64_t img_pg = ho * wo * p->groups;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);

  hipError_t e = hipSuccess;
  dcn::BwdParams b{};
  b.f = geometry(p, ho, wo);
  // The whole-map kernel writes every grad_input element itself, in the I/O
  // dtype: no clear, no rounding pass (16-bit: the workspace only takes the
  // items that fall back to fp32 atomics).  Decided once, before any launch.
  const bool whole_map = dcn::backward_takes_map(b.f);
  if (wide && !whole_map) {
    e = dcn::launch_zero(grad_input, (uint64_t)(p->n * img_in), stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  for (int64_t n0 = 0; n0 < p->n; n0 += per) {
    const int64_t nc = (p->n - n0 < per) ? p->n - n0 : per;
    b.f.input = static_cast<const char *>(input) + n0 * img_in;
    b.f.offset = static_cast<const char *>(offset) + n0 * img_pg * K * 2 * eb;
    b.f.mask = static_cast<const char *>(mask) + n0 * img_pg * K * eb;
    b.f.output = nullptr;
    b.f.in_bytes = (uint32_t)(nc * img_in);
    b.f.off_bytes = (uint32_t)(nc * img_pg * K * 2 * eb);
    b.f.mask_bytes = (uint32_t)(nc * img_pg * K * eb);
    b.f.out_bytes = 0;
    b.f.pg_total = (uint32_t)(nc * img_pg);
    b.grad_out = static_cast<const char *>(grad_output) + n0 * img_pg * dcn::kGroupChannels * eb;
    b.grad_offset = static_cast<char *>(grad_offset) + n0 * img_pg * K * 2 * eb;
    b.grad_mask = static_cast<char *>(grad_mask) + n0 * img_pg * K * eb;
    if (whole_map) {
      b.grad_in = static_cast<char *>(grad_input) + n0 * img_in;
      b.acc = wide ? b.grad_in : ws;
    } else if (wide) {
      b.grad_in = static_cast<char *>(grad_input) + n0 * img_in;
    } else {  // each chunk reuses the accumulator: zero it, accumulate, round out
      b.grad_in = ws;
      e = dcn::launch_zero(ws, (uint64_t)(nc * img_elems * 4), stream);
      if (e != hipSuccess) return hip_fail(e);
    }
    e = dcn::launch_backward(p->dtype, p->softmax, b, whole_map, stream);
    if (e != hipSuccess) return hip_fail(e);
    if (!wide && !whole_map) {
      e = dcn::launch_narrow(p->dtype, ws, static_cast<char *>(grad_input) + n0 * img_in,
                             (uint64_t)(nc * img_elems), stream);
      if (e != hipSuccess) return hip_fail(e);
    }
  }
  return DCN_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_lock;

int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return DCN_ERR_UNSUPPORTED;
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> hold(g_scratch_lock);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e);
      if (!ptr) return hip_fail(hipErrorInvalidSymbol);
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return DCN_OK;
}

}  // namespace

extern "C" {

int dcn_abi_version(void) { return DCN_ABI_VERSION; }

int dcn_check(const dcn_problem *p, int64_t *ho, int64_t *wo) { return validate(p, ho, wo); }

int dcn_forward(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                void *output, void *hip_stream) {
  int64_t ho = 0, wo = 0;
  const int st = validate(p, &ho, &wo);
  if (st != DCN_OK) return st;
  if (p->n == 0) return DCN_OK;
  if (!input || !offset || !mask || !output) return DCN_ERR_NULL;
  if (!aligned16(input) || !aligned16(offset) || !aligned16(mask) || !aligned16(output))
    return DCN_ERR_ALIGN;

  const int eb = elem_bytes(p->dtype);
  const int64_t K = npoints(p);
  const int64_t img_in = (int64_t)p->h * p->w * p->c * eb;
  const int64_t img_pg = ho * wo * p->groups;
  const int64_t per = images_per_chunk(p, ho, wo);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  dcn::FwdParams f = geometry(p, ho, wo);
  for (int64_t n0 = 0; n0 < p->n; n0 += per) {
    const int64_t nc = (p->n - n0 < per) ? p->n - n0 : per;
    f.input = static_cast<const char *>(input) + n0 * img_in;
    f.offset = static_cast<const char *>(offset) + n0 * img_pg * K * 2 * eb;
    f.mask = static_cast<const char *>(mask) + n0 * img_pg * K * eb;
    f.output = static_cast<char *>(output) + n0 * img_pg * dcn::kGroupChannels * eb;
    f.in_bytes = (uint32_t)(nc * img_in);
    f.off_bytes = (uint32_t)(nc * img_pg * K * 2 * eb);
    f.mask_bytes = (uint32_t)(nc * img_pg * K * eb);
    f.out_bytes = (uint32_t)(nc * img_pg * dcn::kGroupChannels * eb);
    f.pg_total = (uint32_t)(nc * img_pg);
    const hipError_t e = dcn::launch_forward(p->dtype, p->softmax, f, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return DCN_OK;
}

int dcn_forward_generated(const dcn_problem *p, int32_t guide_channels, const void *input, const void *guide,
                          const void *w_offset, const void *b_offset, const void *w_mask, const void *b_mask,
                          void *output, void *hip_stream) {
  int64_t ho = 0, wo = 0;
  const int st = validate(p, &ho, &wo);
  if (st != DCN_OK) return st;
  if (guide_channels <= 0 || guide_channels % 8 != 0) return DCN_ERR_SHAPE;
  const int eb = elem_bytes(p->dtype);
  const int64_t K = npoints(p);
  const int64_t img_guide = ho * wo * guide_channels * eb;
  const int64_t w_off_bytes = p->groups * K * 2 * guide_channels * eb;
  if (img_guide > kMaxBytes31 || w_off_bytes > kMaxBytes31) return DCN_ERR_TOO_LARGE;
  if (!dcn::fused_fits(p->groups, (int)K, p->c, false)) return DCN_ERR_UNSUPPORTED;
  if (p->n == 0) return DCN_OK;
  if (!input || !guide || !w_offset || !w_mask || !output) return DCN_ERR_NULL;
  if (!aligned16(input) || !aligned16(guide) || !aligned16(w_offset) || !aligned16(w_mask) || !aligned16(output) ||
      !aligned_elem(b_offset, eb) || !aligned_elem(b_mask, eb))
    return DCN_ERR_ALIGN;

  dcn::FusedParams fp{};
  fp.f = geometry(p, ho, wo);
  fp.cgd = guide_channels;
  fp.w_off = w_offset;
  fp.b_off = b_offset;
  fp.w_mask = w_mask;
  fp.b_mask = b_mask;
  fp.w_off_bytes = (uint32_t)w_off_bytes;
  fp.w_mask_bytes = (uint32_t)(w_off_bytes / 2);
  const int64_t img_in = (int64_t)p->h * p->w * p->c * eb;
  const int64_t img_pix = ho * wo;
  int64_t per = images_per_chunk(p, ho, wo);
  if (kMaxBytes31 / img_guide < per) per = kMaxBytes31 / img_guide;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  for (int64_t n0 = 0; n0 < p->n; n0 += per) {
    const int64_t nc = (p->n - n0 < per) ? p->n - n0 : per;
    fp.f.input = static_cast<const char *>(input) + n0 * img_in;
    fp.f.output = static_cast<char *>(output) + n0 * img_pix * p->c * eb;
    fp.f.in_bytes = (uint32_t)(nc * img_in);
    fp.f.out_bytes = (uint32_t)(nc * img_pix * p->c * eb);
    fp.f.pg_total = (uint32_t)(nc * img_pix * p->groups);
    fp.guide = static_cast<const char *>(guide) + n0 * img_guide;
    fp.guide_bytes = (uint32_t)(nc * img_guide);
    fp.npix = (uint32_t)(nc * img_pix);
    const hipError_t e = dcn::launch_forward_generated(p->dtype, p->softmax, fp, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return DCN_OK;
}

int dcn_forward_projected(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                          const void *w_out, const void *b_out, void *output, void *hip_stream) {
  int64_t ho = 0, wo = 0;
  const int st = validate(p, &ho, &wo);
  if (st != DCN_OK) return st;
  const int eb = elem_bytes(p->dtype);
  const int64_t K = npoints(p);
  const int64_t w_out_bytes = (int64_t)p->c * p->c * eb;
  if (w_out_bytes > kMaxBytes31) return DCN_ERR_TOO_LARGE;
  if (!dcn::fused_fits(p->groups, (int)K, p->c, true)) return DCN_ERR_UNSUPPORTED;
  if (p->n == 0) return DCN_OK;
  if (!input || !offset || !mask || !w_out || !output) return DCN_ERR_NULL;
  if (!aligned16(input) || !aligned16(offset) || !aligned16(mask) || !aligned16(w_out) || !aligned16(output) ||
      !aligned_elem(b_out, eb))
    return DCN_ERR_ALIGN;

  dcn::FusedParams fp{};
  fp.f = geometry(p, ho, wo);
  fp.w_out = w_out;
  fp.b_out = b_out;
  fp.w_out_bytes = (uint32_t)w_out_bytes;
  const int64_t img_in = (int64_t)p->h * p->w * p->c * eb;
  const int64_t img_pix = ho * wo;
  const int64_t img_pg = img_pix * p->groups;
  const int64_t per = images_per_chunk(p, ho, wo);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  for (int64_t n0 = 0; n0 < p->n; n0 += per) {
    const int64_t nc = (p->n - n0 < per) ? p->n - n0 : per;
    fp.f.input = static_cast<const char *>(input) + n0 * img_in;
    fp.f.offset = static_cast<const char *>(offset) + n0 * img_pg * K * 2 * eb;
    fp.f.mask = static_cast<const char *>(mask) + n0 * img_pg * K * eb;
    fp.f.output = static_cast<char *>(output) + n0 * img_pix * p->c * eb;
    fp.f.in_bytes = (uint32_t)(nc * img_in);
    fp.f.off_bytes = (uint32_t)(nc * img_pg * K * 2 * eb);
    fp.f.mask_bytes = (uint32_t)(nc * img_pg * K * eb);
    fp.f.out_bytes = (uint32_t)(nc * img_pix * p->c * eb);
    fp.f.pg_total = (uint32_t)(nc * img_pg);
    fp.npix = (uint32_t)(nc * img_pix);
    const hipError_t e = dcn::launch_forward_projected(p->dtype, p->softmax, fp, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return DCN_OK;
}

int dcn_backward_workspace_size(const dcn_problem *p, uint64_t *bytes) {
  int64_t ho = 0, wo = 0;
  const int st = validate_backward(p, &ho, &wo);
  if (st != DCN_OK) return st;
  if (!bytes) return DCN_ERR_NULL;
  *bytes = workspace_bytes_bwd(p, ho, wo);
  return DCN_OK;
}

int dcn_backward(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                 const void *grad_output, void *grad_input, void *grad_offset, void *grad_mask,
                 void *workspace, uint64_t workspace_bytes, void *hip_stream) {
  int64_t ho = 0, wo = 0;
  const int st = validate_backward(p, &ho, &wo);
  if (st != DCN_OK) return st;
  if (p->n == 0) return DCN_OK;
  const bool wide = p->dtype == DCN_F32;  // grad_input accumulates in place
  if (!wide && !workspace) return DCN_ERR_NULL;
  if (!wide && !aligned16(workspace)) return DCN_ERR_ALIGN;
  if (!wide && workspace_bytes < workspace_bytes_bwd(p, ho, wo)) return DCN_ERR_WORKSPACE;
  return run_backward(p, ho, wo, input, offset, mask, grad_output, grad_input, grad_offset, grad_mask,
                      workspace, images_per_chunk_bwd(p, ho, wo), hip_stream);
}

int dcn_backward_noalloc(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                         const void *grad_output, void *grad_input, void *grad_offset, void *grad_mask,
                         void *hip_stream) {
  int64_t ho = 0, wo = 0;
  const int st = validate_backward(p, &ho, &wo);
  if (st != DCN_OK) return st;
  if (p->n == 0) return DCN_OK;
  int64_t per = images_per_chunk_bwd(p, ho, wo);
  void *ws = nullptr;
  if (p->dtype != DCN_F32) {
    const int64_t img32 = (int64_t)p->h * p->w * p->c * 4;
    if (img32 > (int64_t)kScratchBytes) return DCN_ERR_SCRATCH;
    if ((int64_t)kScratchBytes / img32 < per) per = (int64_t)kScratchBytes / img32;
    const int sst = scratch_address(&ws);
    if (sst != DCN_OK) return sst;
  }
  return run_backward(p, ho, wo, input, offset, mask, grad_output, grad_input, grad_offset, grad_mask, ws,
                      per, hip_stream);
}

const char *dcn_status_string(int status) {
  switch (status) {
    case DCN_OK: return "ok";
    case DCN_ERR_NULL: return "null pointer for a problem or a non-empty tensor";
    case DCN_ERR_SHAPE: return "invalid shape (dims, C % groups, kernel/stride/dilation/pad, or empty output)";
    case DCN_ERR_UNSUPPORTED: return "unsupported dtype, channels per group or point count";
    case DCN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case DCN_ERR_TOO_LARGE: return "a size exceeds the 32-bit index range of one image";
    case DCN_ERR_HIP: return g_hip_message;
    case DCN_ERR_ABI: return "dcn_problem.struct_size does not match this library";
    case DCN_ERR_ARG: return "invalid argument value (softmax or remove_center flag, or offset_scale)";
    case DCN_ERR_WORKSPACE: return "workspace smaller than dcn_backward_workspace_size reports";
    case DCN_ERR_SCRATCH: return "dcn_backward_noalloc: one image's fp32 grad_input accumulator exceeds the library's fixed scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
