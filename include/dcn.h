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
 *   index sits at grid index k + 1) and the softmax runs over those K.  Ho = (H + 2*pad_h - dilation_h*(kernel_h-1) - 1)/stride_h + 1
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
 * are fp32 for every I/O dtype; 16-bit results are rounded to nearest-even.
 *
 * Ownership and execution: every tensor pointer is a DEVICE pointer owned by
 * the caller.  The library allocates nothing, keeps no pointer after it
 * returns and has no mutable global state, so calls are reentrant.  Work is
 * enqueued on the caller's hipStream_t (NULL = the null stream) and the call
 * returns without waiting: DCN_OK means "validated and enqueued".  Outputs are
 * overwritten, never accumulated into, and must not alias any input.
 *
 * Kernel choice: the forward picks its kernel from the problem (dtype, point
 * count, stride, dilation, map and window size; the forward with
 * remove_center runs the untiled kernel).  The environment variable
 * DCN_MI355X_FWD_PATH = "generic" | "tiled" (one group per work item) |
 * "pair" (two groups per work item) | "lane" | "map" (whole maps in LDS),
 * read at every call, makes it try that kernel first; DCN_MI355X_BWD_PATH =
 * "generic" | "tiled" (half windows) | "quad" does the same for the
 * backward.  Results agree to rounding either way.
 *
 * Errors: every entry point returns DCN_OK (0) or a negative dcn_status.
 * Nothing is enqueued when a check fails.  N == 0 is valid and enqueues
 * nothing.  There is no fallback path: an unsupported problem is an error.
 */
#ifndef DCN_MI355X_H
#define DCN_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCN_ABI_VERSION 3

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
                                 without a kernel, or a 16-bit backward other than
                                 3x3 points at stride 1, dilation 1 or 2               */
    DCN_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned                */
    DCN_ERR_TOO_LARGE = -5,   /* one image's input, output or offset tensor exceeds
                                 2^31-1 bytes, or H or W exceeds 2^24 (16-bit
                                 backward: also H*W*C*4 bytes, its fp32 accumulator)   */
    DCN_ERR_HIP = -6,         /* the HIP runtime refused a launch; see dcn_status_string */
    DCN_ERR_ABI = -7,         /* problem->struct_size != sizeof(dcn_problem)            */
    DCN_ERR_ARG = -8,         /* softmax or remove_center not 0/1, remove_center with
                                 an even kernel size, or offset_scale not finite       */
    DCN_ERR_WORKSPACE = -9    /* dcn_backward's workspace_bytes below what
                                 dcn_backward_workspace_size reports                   */
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
 * right (the floor convention).  fp32 for every shape.  16-bit I/O (all
 * tensors of the call in that dtype) for 3x3 points (remove_center or not)
 * at stride 1 and dilation 1 or 2 (equal on both axes), else
 * DCN_ERR_UNSUPPORTED.  The arithmetic is fp32 throughout and grad_input
 * is accumulated in fp32: sums per output tile in fixed point, added with
 * fp32 atomics (so its low bits can vary from run to run).  For fp32 the sums
 * land in grad_input itself (the call zeroes it first) and workspace may be
 * NULL.  For 16-bit I/O they land in `workspace`, a caller-owned device
 * buffer of at least dcn_backward_workspace_size bytes, 16-byte aligned, whose
 * contents on entry do not matter and are garbage on return; each chunk of
 * images zeroes it, accumulates into it and is then rounded once to
 * nearest-even into grad_input, like grad_offset and grad_mask.  Calls that
 * share a workspace must be ordered on one stream.
 * Enqueues per chunk of images a fill kernel, one backward launch and, for
 * 16-bit I/O, one rounding kernel (fp32: one fill for the whole batch). */
int dcn_backward(const dcn_problem *p, const void *input, const void *offset, const void *mask,
                 const void *grad_output, void *grad_input, void *grad_offset, void *grad_mask,
                 void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* Static description of a status code.  For DCN_ERR_HIP the string carries
 * the HIP runtime's message from the calling thread's most recent failure. */
const char *dcn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DCN_MI355X_H */
