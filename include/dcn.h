/*
 * dcn.h -- C ABI of the MI355X (gfx950) DCNv3/DCNv4 deformable-sampling core.
 *
 * The operation (defined on the page wmrh.cn/news/61976, "internimage_l_22k_384
 * / DCNv3 core operator explained", section 二 steps 2-4 and section 三; the
 * unnormalised DCNv4 variant and the NHWC layout on pnsm.cn/news/2029644.html,
 * sections 2.2-2.3 and 3.3):
 *
 *   for every image n, output pixel (ho, wo), group g and kernel point
 *   k = i*kernel_w + j (i along H, j along W), K = kernel_h*kernel_w points:
 *     py  = ho*stride_h - pad_h + i*dilation_h + offset_scale * offset[n,ho,wo,g,k,1]
 *     px  = wo*stride_w - pad_w + j*dilation_w + offset_scale * offset[n,ho,wo,g,k,0]
 *     m_k = softmax_k(mask[n,ho,wo,g,:])   if softmax != 0   (DCNv3)
 *         = mask[n,ho,wo,g,k]              if softmax == 0   (DCNv4)
 *     out[n,ho,wo,g*Cg+c] = sum_k m_k * bilinear(input[n,:,:,g*Cg+c], py, px)
 *
 *   bilinear() puts pixel centres at integer coordinates and reads zero outside
 *   [0,H) x [0,W).
 *
 *   remove_center (DCNv4's option of that name, pnsm.cn/news/2029644.html
 *   section 3.3; odd kernel sizes only) drops the centre point (i, j) =
 *   (kernel_h/2, kernel_w/2): K = kernel_h*kernel_w - 1, the points keep the
 *   row-major order with the centre skipped (point k at or past the centre's
 *   index sits at grid index k + 1) and the softmax runs over those K.
 *
 *   Output extent (the convolution arithmetic behind the pages' statements
 *   that pad = kernel_size // 2 keeps a stride-1 output at the input's size,
 *   pnsm.cn/news/2029644.html section 3.3 and trdm.cn/news/584307, "DCNv3
 *   operator compilation", section 2.3):
 *     Ho = (H + 2*pad_h - dilation_h*(kernel_h-1) - 1) / stride_h + 1
 *   (integer division; the same form gives Wo).  Cg = C / groups.
 *
 * Layouts (all tensors dense and contiguous, row-major, one dtype per call):
 *   input        (N, H, W, C)                              NHWC
 *   offset       (N, Ho, Wo, groups, K, 2)                 pair stored (x, y)
 *   mask         (N, Ho, Wo, groups, K)                    logits or weights
 *   output       (N, Ho, Wo, C)                            NHWC
 *   grad_*       the shape of the tensor it is the gradient of.
 *
 * Arithmetic: sampling locations, weights, the softmax and every accumulation
 * are fp32 for every I/O dtype (the tiled and whole-map backward kernels sum
 * grad_input in exact integer arithmetic on a per-item fixed-point grid
 * instead, with the error bound stated at dcn_backward); 16-bit results are
 * rounded to nearest-even.
 *
 * Ownership and execution: every tensor pointer is a DEVICE pointer owned by
 * the caller.  dcn_forward and dcn_backward allocate nothing, keep no
 * pointer after they return and touch no mutable global state, so calls are
 * reentrant (dcn_backward_noalloc's fixed scratch is the one exception; see
 * there).  Work is enqueued on the caller's hipStream_t (NULL = the null
 * stream) and the call returns without waiting: DCN_OK means "validated and
 * enqueued".  Outputs are overwritten, never accumulated into, and must not
 * alias any input.
 *
 * Kernel choice (3x3 points unless noted): output maps smaller than one
 * 16x16 tile, or that such tiles would leave over half empty, run the
 * whole-map kernel; other maps whose tile window fits the LDS run a tiled
 * kernel (fp32: the quad kernel, two groups per work item where the group
 * count is even, at stride 1 or 2 and dilation 1 or 2, with or without the
 * centre; 16-bit I/O: the lane kernel, up to four groups per work item, at
 * stride and dilation 1, else the quad kernel); 5x5 points at stride and
 * dilation 1 run the lane kernel in every dtype; everything else (other
 * point sets, windows that do not fit) runs the untiled kernel.  The
 * backward runs the whole-map kernel for 3x3 points at dilation 1 where the
 * input and output maps both fit 12x12, 16x16 or 24x24 at stride 1, or the
 * input fits 24x24 at stride 2 (one work item per image and group), the
 * tiled quad kernel for other 3x3 problems at
 * stride 1 or 2 and dilation 1 or 2 and for 5x5 points at stride and
 * dilation 1, else the untiled kernel.  The environment variable
 * DCN_MI355X_FWD_PATH = "generic" | "tiled" (one group per work item) |
 * "pair" (two groups per work item) | "lane" | "map" (whole maps in LDS),
 * read at every call, makes the forward try that kernel first;
 * DCN_MI355X_BWD_PATH = "generic" | "tiled" (half windows, fp32) | "quad" |
 * "map" does the same for the backward.  Results agree to rounding either
 * way.
 *
 * Errors: every entry point returns DCN_OK (0) or a negative dcn_status.
 * Nothing is enqueued when a check fails (every check of the problem, the
 * pointers and the workspace runs before the first launch).  A DCN_ERR_HIP
 * from a launch can come after earlier launches of the same call (a chunk,
 * or the grad_input clear) were enqueued: the outputs are then partly
 * written and must be discarded.  N == 0 is valid and enqueues nothing.
 * There is no fallback path: an unsupported problem is an error.
 */
#ifndef DCN_MI355X_H
#define DCN_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCN_ABI_VERSION 6

/* Bytes of the fixed device scratch behind dcn_backward_noalloc (one copy
 * per GPU the library runs on, held until the process ends). */
#define DCN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Element type of every tensor of one call. */
typedef enum dcn_dtype {
    DCN_F32 = 0,
    DCN_F16 = 1,
    DCN_BF16 = 2
} dcn_dtype;

typedef enum dcn_status {
    DCN_OK = 0,
    DCN_ERR_NULL = -1,        /* NULL problem, or NULL pointer for a non-empty tensor   */
    DCN_ERR_SHAPE = -2,       /* a dim <= 0 (N may be 0), C % groups != 0, kernel,
                                 stride or dilation < 1, pad < 0, Ho/Wo < 1, or no
                                 point left (1x1 with remove_center)                   */
    DCN_ERR_UNSUPPORTED = -3, /* dtype, channels-per-group or point count (K > 64)
                                 without a kernel                                      */
    DCN_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned                */
    DCN_ERR_TOO_LARGE = -5,   /* one image's input, output or offset tensor exceeds
                                 2^31-1 bytes, or H or W exceeds 2^24 (16-bit
                                 backward: also H*W*C*4 bytes, its fp32 accumulator)   */
    DCN_ERR_HIP = -6,         /* the HIP runtime refused a launch; see dcn_status_string */
    DCN_ERR_ABI = -7,         /* problem->struct_size != sizeof(dcn_problem)            */
    DCN_ERR_ARG = -8,         /* softmax or remove_center not 0/1, remove_center with
                                 an even kernel size, or offset_scale not finite       */
    DCN_ERR_WORKSPACE = -9,   /* dcn_backward's workspace_bytes below what
                                 dcn_backward_workspace_size reports                   */
    DCN_ERR_SCRATCH = -10     /* dcn_backward_noalloc, 16-bit I/O: one image's fp32
                                 grad_input accumulator (H*W*C*4 bytes) exceeds
                                 DCN_NOALLOC_SCRATCH_BYTES                             */
} dcn_status;

/* One problem description.  Set struct_size = sizeof(dcn_problem). */
typedef struct dcn_problem {
    uint32_t struct_size;
    int32_t n, h, w, c, groups;
    int32_t kernel_h, kernel_w;
    int32_t stride_h, stride_w;
    int32_t pad_h, pad_w;
    int32_t dilation_h, dilation_w;
    float offset_scale;   /* multiplies the learned offset only, not the grid   */
    int32_t softmax;      /* 1 = DCNv3 (softmax over the points), 0 = DCNv4     */
    int32_t dtype;        /* dcn_dtype                                          */
    int32_t remove_center;/* 1 = the kernel's centre point is not sampled       */
} dcn_problem;

/* Version of this ABI (DCN_ABI_VERSION of the built library). */
int dcn_abi_version(void);

/* Validate a problem on the host (no device call) and report the output
 * extent.  ho / wo may be NULL.  Returns DCN_OK or the first failing check
 * (also for problems that dcn_forward could not run: unsupported dtype,
 * channels per group or point count, or sizes beyond the index width). */
int dcn_check(const dcn_problem *p, int64_t *ho, int64_t *wo);

/* Forward: output = DCN(input, offset, mask).  Enqueues one kernel launch per
 * chunk of images (one chunk unless an image batch exceeds 2 GiB of input). */
int dcn_forward(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                void *output, void *hip_stream);

/* The forward with the step before the core fused in (wmrh.cn/news/61976,
 * section 二 steps 2 and 3: a linear layer of the guide feature gives every
 * point's (x, y) offset per group, the other branch of the same linear
 * structure its score): for every output pixel q and group g,
 *   offset[q, g, k, e] = sum_c guide[q, c] * w_offset[(g*K + k)*2 + e, c] + b_offset[(g*K + k)*2 + e]
 *   mask[q, g, k]      = sum_c guide[q, c] * w_mask[g*K + k, c]          + b_mask[g*K + k]
 * and then output = DCN(input, offset, mask) as dcn_forward computes it
 * (softmax over the K mask values when p->softmax).  The offsets and mask
 * values are formed on the matrix cores with fp32 accumulation, kept in
 * fp32 and never stored.
 *   guide     (N, Ho, Wo, guide_channels), guide_channels a positive multiple of 8
 *   w_offset  (groups*K*2, guide_channels), row-major (out, in)
 *   b_offset  (groups*K*2) or NULL (no bias)
 *   w_mask    (groups*K, guide_channels), b_mask (groups*K) or NULL
 * Every tensor is in p->dtype; input, guide, the weights and output 16-byte
 * aligned.  Errors as dcn_forward, plus DCN_ERR_SHAPE for guide_channels and
 * DCN_ERR_UNSUPPORTED when one group's generated values do not fit the
 * kernel's LDS.  Enqueues one launch per chunk of images.
 * Throughput: the fused kernel gathers its corners from global memory (its
 * blocks own a few pixels with all their groups, where the sampling kernels
 * stage one tile's window of one or a few groups), so on MI355X at the
 * InternImage stage shapes this call takes about twice as long as a
 * library GEMM for the two branches followed by dcn_forward.  It is for
 * callers that must not hold the offset and mask tensors. */
int dcn_forward_generated(const dcn_problem *p, int32_t guide_channels, const void *input, const void *guide,
                          const void *w_offset, const void *b_offset, const void *w_mask, const void *b_mask,
                          void *output, void *hip_stream);

/* The forward with the step after the core fused in (wmrh.cn/news/61976,
 * section 二 step 4: the weighted sum passes through the output_proj linear
 * layer): output[q, o] = sum_c y[q, c] * w_out[o, c] + b_out[o], where y is
 * what dcn_forward computes, kept in fp32 on chip; the product runs on the
 * matrix cores with fp32 accumulation (for 16-bit I/O y enters them as two
 * parts in p->dtype, its rounding and the rounding of the remainder, which
 * keeps about twice the dtype's significant bits of y).
 *   w_out (C, C), row-major (out, in); b_out (C) or NULL.
 * Layouts, errors and chunking otherwise as dcn_forward
 * (DCN_ERR_UNSUPPORTED when the kernel's LDS cannot hold 16 pixels of C
 * channels).
 * Throughput: each block of 16 pixels reads all of w_out for its one
 * matrix-core row tile and gathers its corners from global memory, so this
 * call is 2.5x (C = 160) to 16x (C = 1280) slower on MI355X than
 * dcn_forward followed by a library GEMM; it is for callers that must not
 * hold the core's output before the projection. */
int dcn_forward_projected(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                          const void *w_out, const void *b_out, void *output, void *hip_stream);

/* Bytes of device workspace that dcn_backward needs for this problem: 0 for
 * fp32 (and for N == 0); for 16-bit I/O, one fp32 grad_input accumulator of
 * the largest chunk of images (N*H*W*C*4 bytes unless the batch is split).
 * Runs the backward's checks (the errors dcn_backward would return before
 * touching a pointer); bytes must not be NULL. */
int dcn_backward_workspace_size(const dcn_problem *p, uint64_t *bytes);

/* Backward of the forward above for the gradient grad_output of output:
 *   grad_input  = adjoint bilinear scatter of m_k * weight * grad_output,
 *   grad_offset = offset_scale * m_k * sum_c grad_output_c * d(bilinear)/d(px, py),
 *                 stored (x, y) like the offsets,
 *   grad_mask   = gradient with respect to the mask tensor as passed: through
 *                 the softmax Jacobian when softmax != 0.
 * At integer sampling coordinates the derivative is the one-sided one from the
 * right (the floor convention).  Every shape, in fp32 and in 16-bit I/O (all
 * tensors of the call in that dtype).  The arithmetic is fp32 throughout and
 * grad_input is accumulated in fp32 atomics, so its low bits can vary from
 * run to run.  The tiled quad kernel (the shapes under kernel choice above)
 * first sums each output tile's scatter in fixed point on the tile's own grid: a
 * term is rounded to a multiple of 2^(e-30), where 2^e bounds the tile's sum
 * B of sum_k |m_k| * max_c |grad_output_c| over its pixel-groups, so an
 * element reached by n terms is off by at most n * 2^(e-31) <= n * B * 2^-30.
 * A tile whose B exceeds 2^12 times its smallest nonzero per-pixel-group term
 * (an outlier in grad_output or the mask), or is not finite, adds its terms
 * with fp32 atomics instead; so the fixed-point error of an element stays
 * within n * 2^-18 of the term bound of every pixel-group that reaches it.
 * For fp32 the sums
 * land in grad_input itself (the call zeroes it first) and workspace may be
 * NULL.  For 16-bit I/O they land in `workspace`, a caller-owned device
 * buffer of at least dcn_backward_workspace_size bytes, 16-byte aligned, whose
 * contents on entry do not matter and are garbage on return; each chunk of
 * images zeroes it, accumulates into it and is then rounded once to
 * nearest-even into grad_input, like grad_offset and grad_mask.  Calls that
 * share a workspace must be ordered on one stream.
 * The whole-map kernel applies the same fixed point with one grid per
 * (image, group), whose whole grad_input slice it owns: it writes that slice
 * once, rounded to the I/O dtype, so grad_input is not zeroed first and an
 * item on fixed point gives the same bits from run to run; the workspace
 * (still required for 16-bit I/O) only takes the items that fall back to
 * fp32 atomics, each clearing its own slice of it first (fp32: grad_input
 * itself).
 * Enqueues per chunk of images a fill kernel, one backward launch and, for
 * 16-bit I/O, one rounding kernel (fp32: one fill for the whole batch);
 * for the whole-map kernel's shapes only the backward launch. */
int dcn_backward(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                 const void *grad_output, void *grad_input, void *grad_offset, void *grad_mask,
                 void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* dcn_backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same checks, kernels and results as dcn_backward, with the 16-bit fp32
 * grad_input accumulator in a fixed device scratch the library owns
 * (DCN_NOALLOC_SCRATCH_BYTES on each GPU, part of the library's device code,
 * so the HIP runtime reserves it when it loads that code) instead of a caller
 * workspace.  The batch runs in chunks of images whose accumulator fits the
 * scratch (so possibly more chunks than dcn_backward); each chunk clears it with a fill
 * kernel, so whatever a previous call left there does not matter.  16-bit
 * I/O with one image's accumulator (H*W*C*4 bytes) above the scratch returns
 * DCN_ERR_SCRATCH before enqueueing anything.  fp32 needs no scratch and
 * behaves exactly like dcn_backward without a workspace.  The call allocates
 * nothing: the scratch's device address is looked up once per device, on the
 * first call made with that device current, and kept.
 * Every call on one GPU shares that GPU's scratch: 16-bit calls that may
 * overlap on the device (other streams, other host threads) race and must be
 * ordered by the caller, for instance on one stream. */
int dcn_backward_noalloc(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                         const void *grad_output, void *grad_input, void *grad_offset, void *grad_mask,
                         void *hip_stream);

/* Static description of a status code.  For DCN_ERR_HIP the string carries
 * the HIP runtime's message from the calling thread's most recent failure. */
const char *dcn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DCN_MI355X_H */
