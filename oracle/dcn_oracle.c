/*
 * dcn_oracle.c -- plain, slow fp64 CPU oracle for the DCNv3/DCNv4 deformable
 * sampling core.  TEST INFRASTRUCTURE ONLY: it is linked by the test-suite, by
 * the smoke check and by the benchmark's CPU-baseline leg, never by the
 * product path.  It shares no source, header or helper with the HIP library.
 *
 * Pages cited (addresses as printed on them):
 *   [P5] wmrh.cn/news/61976, "internimage_l_22k_384 / DCNv3 core operator
 *        explained": section 二 (the four steps of a DCNv3 forward), the
 *        "细节亮点" note (zero-initialised offset/mask), section 三
 *        (offset_scale = 2.0).
 *   [P2] pnsm.cn/news/2029644.html, "FlashInternImage / DCNv4": section 2.3
 *        (NHWC output layout), section 3.3 (pad = kernel_size // 2).
 *   [P4] trdm.cn/news/584307, "DCNv3 operator compilation": section 2.3
 *        (stride-1 output keeps the input's spatial size).
 *   [P2 §3.3] also lists DCNv4's remove_center argument: the kernel's centre
 *        point is dropped from the sampling set.
 *
 * What is computed (the operation as the pages define it, written out):
 *   For every image n, output pixel (ho, wo), group g and kernel point
 *   k = i*KW + j (i along H, j along W):
 *     py = ho*stride_h - pad_h + i*dil_h + s * off[n,ho,wo,g,k,1]
 *     px = wo*stride_w - pad_w + j*dil_w + s * off[n,ho,wo,g,k,0]
 *   [P5 §二 step 2: one (x, y) offset per point and group; §三: the offset is
 *   multiplied by offset_scale s before it moves the point off the regular
 *   3x3 grid].
 *     m_k = softmax over the K points of mask[n,ho,wo,g,:]       (DCNv3,
 *           [P5 §二 step 3]), or m_k = mask[n,ho,wo,g,k]           (DCNv4).
 *     y[n,ho,wo,g*Cg+c] = sum_k m_k * B(X[n,:,:,g*Cg+c], py, px)
 *   [P5 §二 step 4: per group, bilinear sampling then mask-weighted sum].
 *   B is bilinear interpolation with pixel centres at integer coordinates and
 *   zero outside [0,H) x [0,W):
 *     B(X, py, px) = sum_{yc in {y0,y0+1}, xc in {x0,x0+1}}
 *                      (1-|py-yc|) * (1-|px-xc|) * Xz[yc, xc],
 *     y0 = floor(py), x0 = floor(px), Xz = X inside the map, 0 outside.
 *   With remove_center (odd KH and KW) the centre point (i, j) = (KH/2, KW/2)
 *   is left out: K = KH*KW - 1 points, numbered in the same row-major order
 *   with the centre skipped (point k >= KH/2*KW + KW/2 sits at grid index
 *   k + 1), and the DCNv3 softmax runs over those K points only.
 *   Layouts: x and y are NHWC with C = G*Cg [P2 §2.3]; offsets are
 *   (N,Ho,Wo,G,K,2) with the pair stored as (x, y); mask is (N,Ho,Wo,G,K),
 *   K = KH*KW (KH*KW - 1 with remove_center).
 *   Ho = floor((H + 2*pad_h - dil_h*(KH-1) - 1)/stride_h) + 1 (same for Wo).
 *
 * Backward (the exact derivatives of the definition above, one-sided from the
 * right at integer coordinates, i.e. the floor convention):
 *   dL/dX     : adjoint of the bilinear gather (scatter of m_k*w*gy),
 *   dL/doff   : s * m_k * sum_c gy_c * dB/d(px|py),
 *   dL/dmask  : gm_k = sum_c gy_c * B_k[c]; for DCNv3 through the softmax
 *               Jacobian, gl_k = m_k * (gm_k - sum_j m_j gm_j).
 *
 * The steps before and after the core [P5 §二 steps 2-4]: a linear layer of
 * the guide feature gives, per output pixel, the 2K offset components and
 * the K mask values of every group (two branches of the same linear
 * structure, step 2 for the offsets and step 3 for the scores); after the
 * weighted sum, the output_proj linear layer maps the C channels of each
 * pixel to C channels (step 4).  A linear layer here is
 *   out[q, o] = sum_c in[q, c] * W[o, c] + b[o]
 * for every row q (W row-major, out_features x in_features; b optional).
 * The offset rows of W are ordered (g, k, e): row g*K*2 + k*2 + e gives
 * component e (0 = x, 1 = y) of point k of group g; the mask rows (g, k).
 *
 * Non-finite values: a NaN offset makes that sample NaN; an infinite offset
 * puts the sample outside the map, where B = 0, so it contributes m_k * 0
 * (0 for a finite m_k, NaN for a NaN or infinite one, as IEEE arithmetic
 * evaluates the definition).  Arithmetic is fp64
 * throughout; inputs given in 16-bit or fp32 are widened exactly by the
 * caller.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* The oracle's own description of one problem (independent of the HIP
 * library's struct). */
typedef struct {
    int64_t n, h, w, c, groups;
    int64_t kh, kw;
    int64_t stride_h, stride_w;
    int64_t pad_h, pad_w;
    int64_t dil_h, dil_w;
    double offset_scale;
    int64_t softmax; /* 1 = DCNv3 (softmax over the points), 0 = DCNv4 */
    int64_t remove_center; /* 1 = the centre point is not sampled (odd KH, KW) */
} ref_problem;

/* Number of sampling points per (pixel, group). */
static int64_t npoints(const ref_problem *p)
{
    return p->kh * p->kw - (p->remove_center ? 1 : 0);
}

int64_t ref_out_size(int64_t in, int64_t k, int64_t stride, int64_t pad, int64_t dil)
{
    int64_t span = in + 2 * pad - dil * (k - 1) - 1;
    if (stride <= 0 || span < 0)
        return 0;
    return span / stride + 1;
}

/* Feature value with zero outside the map. */
static double feat(const ref_problem *p, const double *x, int64_t n, int64_t yy, int64_t xx,
                   int64_t ch)
{
    if (yy < 0 || yy >= p->h || xx < 0 || xx >= p->w)
        return 0.0;
    return x[((n * p->h + yy) * p->w + xx) * p->c + ch];
}

/* Modulation scalars m_k of one (pixel, group): softmax or identity. */
static void mask_weights(const ref_problem *p, const double *mrow, double *m)
{
    int64_t K = npoints(p);
    if (!p->softmax) {
        for (int64_t k = 0; k < K; ++k)
            m[k] = mrow[k];
        return;
    }
    double mx = mrow[0];
    for (int64_t k = 1; k < K; ++k)
        mx = fmax(mx, mrow[k]);
    double sum = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        m[k] = exp(mrow[k] - mx);
        sum += m[k];
    }
    for (int64_t k = 0; k < K; ++k)
        m[k] /= sum;
}

/* Sampling location of point k of output pixel (ho, wo). */
static void location(const ref_problem *p, int64_t ho, int64_t wo, int64_t k,
                     const double *offk, double *py, double *px)
{
    int64_t q = k; /* position on the KH x KW grid */
    if (p->remove_center && q >= (p->kh / 2) * p->kw + p->kw / 2)
        ++q;
    int64_t i = q / p->kw, j = q % p->kw;
    *py = (double)(ho * p->stride_h - p->pad_h + i * p->dil_h) + p->offset_scale * offk[1];
    *px = (double)(wo * p->stride_w - p->pad_w + j * p->dil_w) + p->offset_scale * offk[0];
}

/* Corner bookkeeping of one bilinear sample.  Returns -1 when the location is
 * NaN, 0 when it is infinitely (or absurdly, beyond 1e15 pixels) far away and
 * so outside the map, 1 otherwise.  Corners outside the map are kept here and
 * read as zero by feat(), so no early exit changes the one-sided derivative
 * at the map's border. */
static int corners(const ref_problem *p, double py, double px, int64_t cy[2], int64_t cx[2],
                   double wy[2], double wx[2])
{
    (void)p;
    if (isnan(py) || isnan(px))
        return -1;
    if (!(fabs(py) < 1e15 && fabs(px) < 1e15))
        return 0;
    double fy = floor(py), fx = floor(px);
    cy[0] = (int64_t)fy;
    cy[1] = cy[0] + 1;
    cx[0] = (int64_t)fx;
    cx[1] = cx[0] + 1;
    for (int a = 0; a < 2; ++a) {
        wy[a] = 1.0 - fabs(py - (double)cy[a]);
        wx[a] = 1.0 - fabs(px - (double)cx[a]);
    }
    return 1;
}

/* One output row of C channels at (n, ho, wo). */
static void forward_pixel(const ref_problem *p, int64_t Ho, int64_t Wo, const double *x,
                          const double *off, const double *mask, int64_t n, int64_t ho,
                          int64_t wo, double *yrow)
{
    int64_t G = p->groups, Cg = p->c / p->groups, K = npoints(p);
    double *m = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t g = 0; g < G; ++g) {
        int64_t pg = ((n * Ho + ho) * Wo + wo) * G + g;
        mask_weights(p, mask + pg * K, m);
        for (int64_t c = 0; c < Cg; ++c)
            yrow[g * Cg + c] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double py, px;
            location(p, ho, wo, k, off + (pg * K + k) * 2, &py, &px);
            int64_t cy[2], cx[2];
            double wy[2], wx[2];
            int st = corners(p, py, px, cy, cx, wy, wx);
            if (st < 0) {
                for (int64_t c = 0; c < Cg; ++c)
                    yrow[g * Cg + c] = NAN;
                continue;
            }
            if (st == 0) { /* B = 0 for a sample infinitely far away */
                for (int64_t c = 0; c < Cg; ++c)
                    yrow[g * Cg + c] += m[k] * 0.0;
                continue;
            }
            for (int64_t c = 0; c < Cg; ++c) {
                double b = 0.0;
                for (int a = 0; a < 2; ++a)
                    for (int e = 0; e < 2; ++e)
                        b += wy[a] * wx[e] * feat(p, x, n, cy[a], cx[e], g * Cg + c);
                yrow[g * Cg + c] += m[k] * b;
            }
        }
    }
    free(m);
}

/* Whole forward: y is (N, Ho, Wo, C). */
void ref_forward(const ref_problem *p, const double *x, const double *off, const double *mask,
                 double *y)
{
    int64_t Ho = ref_out_size(p->h, p->kh, p->stride_h, p->pad_h, p->dil_h);
    int64_t Wo = ref_out_size(p->w, p->kw, p->stride_w, p->pad_w, p->dil_w);
    for (int64_t n = 0; n < p->n; ++n)
        for (int64_t ho = 0; ho < Ho; ++ho)
            for (int64_t wo = 0; wo < Wo; ++wo)
                forward_pixel(p, Ho, Wo, x, off, mask, n, ho, wo,
                              y + ((n * Ho + ho) * Wo + wo) * p->c);
}

/* Forward at selected output pixels only: pix[i] = (n*Ho + ho)*Wo + wo,
 * y is (npix, C).  Used to check full-size runs one output row at a time. */
void ref_forward_pixels(const ref_problem *p, const double *x, const double *off,
                        const double *mask, const int64_t *pix, int64_t npix, double *y)
{
    int64_t Ho = ref_out_size(p->h, p->kh, p->stride_h, p->pad_h, p->dil_h);
    int64_t Wo = ref_out_size(p->w, p->kw, p->stride_w, p->pad_w, p->dil_w);
    for (int64_t i = 0; i < npix; ++i) {
        int64_t q = pix[i];
        int64_t wo = q % Wo, ho = (q / Wo) % Ho, n = q / (Wo * Ho);
        forward_pixel(p, Ho, Wo, x, off, mask, n, ho, wo, y + i * p->c);
    }
}

/* Whole backward.  gx (N,H,W,C), goff (N,Ho,Wo,G,K,2), gmask (N,Ho,Wo,G,K)
 * are overwritten. */
void ref_backward(const ref_problem *p, const double *x, const double *off, const double *mask,
                  const double *gy, double *gx, double *goff, double *gmask)
{
    int64_t Ho = ref_out_size(p->h, p->kh, p->stride_h, p->pad_h, p->dil_h);
    int64_t Wo = ref_out_size(p->w, p->kw, p->stride_w, p->pad_w, p->dil_w);
    int64_t G = p->groups, Cg = p->c / p->groups, K = npoints(p);
    double s = p->offset_scale;
    memset(gx, 0, sizeof(double) * (size_t)(p->n * p->h * p->w * p->c));
    double *m = (double *)malloc(sizeof(double) * (size_t)K);
    double *gm = (double *)malloc(sizeof(double) * (size_t)K);
    for (int64_t n = 0; n < p->n; ++n)
        for (int64_t ho = 0; ho < Ho; ++ho)
            for (int64_t wo = 0; wo < Wo; ++wo)
                for (int64_t g = 0; g < G; ++g) {
                    int64_t pg = ((n * Ho + ho) * Wo + wo) * G + g;
                    const double *gyr = gy + ((n * Ho + ho) * Wo + wo) * p->c + g * Cg;
                    mask_weights(p, mask + pg * K, m);
                    for (int64_t k = 0; k < K; ++k) {
                        double py, px;
                        location(p, ho, wo, k, off + (pg * K + k) * 2, &py, &px);
                        int64_t cy[2], cx[2];
                        double wy[2], wx[2];
                        double *go = goff + (pg * K + k) * 2;
                        int st = corners(p, py, px, cy, cx, wy, wx);
                        gm[k] = 0.0;
                        go[0] = go[1] = 0.0;
                        if (st < 0) {
                            gm[k] = go[0] = go[1] = NAN;
                            continue;
                        }
                        if (st == 0) { /* B = 0 and dB = 0 far away */
                            go[0] = s * m[k] * 0.0;
                            go[1] = s * m[k] * 0.0;
                            continue;
                        }
                        /* d(1-|py-yc|)/dpy: -1 for yc = y0, +1 for yc = y0+1
                         * (one-sided from the right at integers). */
                        const double dsy[2] = {-1.0, 1.0}, dsx[2] = {-1.0, 1.0};
                        double gpy = 0.0, gpx = 0.0;
                        for (int64_t c = 0; c < Cg; ++c) {
                            int64_t ch = g * Cg + c;
                            double b = 0.0, dby = 0.0, dbx = 0.0;
                            for (int a = 0; a < 2; ++a)
                                for (int e = 0; e < 2; ++e) {
                                    double v = feat(p, x, n, cy[a], cx[e], ch);
                                    b += wy[a] * wx[e] * v;
                                    dby += dsy[a] * wx[e] * v;
                                    dbx += wy[a] * dsx[e] * v;
                                    if (cy[a] >= 0 && cy[a] < p->h && cx[e] >= 0 && cx[e] < p->w)
                                        gx[((n * p->h + cy[a]) * p->w + cx[e]) * p->c + ch] +=
                                            m[k] * wy[a] * wx[e] * gyr[c];
                                }
                            gm[k] += gyr[c] * b;
                            gpy += gyr[c] * dby;
                            gpx += gyr[c] * dbx;
                        }
                        go[0] = s * m[k] * gpx;
                        go[1] = s * m[k] * gpy;
                    }
                    double *gmr = gmask + pg * K;
                    if (p->softmax) {
                        double dot = 0.0;
                        for (int64_t k = 0; k < K; ++k)
                            dot += m[k] * gm[k];
                        for (int64_t k = 0; k < K; ++k)
                            gmr[k] = m[k] * (gm[k] - dot);
                    } else {
                        for (int64_t k = 0; k < K; ++k)
                            gmr[k] = gm[k];
                    }
                }
    free(m);
    free(gm);
}

/* A linear layer over `rows` rows: out (rows, nout) = in (rows, nin) times
 * the transpose of w (nout, nin), plus b (nout) when b is not NULL. */
void ref_linear(int64_t rows, int64_t nin, int64_t nout, const double *in, const double *w,
                const double *b, double *out)
{
    for (int64_t q = 0; q < rows; ++q)
        for (int64_t o = 0; o < nout; ++o) {
            double acc = b ? b[o] : 0.0;
            for (int64_t c = 0; c < nin; ++c)
                acc += in[q * nin + c] * w[o * nin + c];
            out[q * nout + o] = acc;
        }
}

/* The core with its offsets and mask generated from a guide feature
 * (N, Ho, Wo, cgd) by the two linear branches w_off (G*K*2, cgd), b_off and
 * w_mask (G*K, cgd), b_mask (biases may be NULL): y is (N, Ho, Wo, C). */
void ref_forward_om(const ref_problem *p, const double *x, const double *guide, int64_t cgd,
                    const double *w_off, const double *b_off, const double *w_mask,
                    const double *b_mask, double *y)
{
    int64_t Ho = ref_out_size(p->h, p->kh, p->stride_h, p->pad_h, p->dil_h);
    int64_t Wo = ref_out_size(p->w, p->kw, p->stride_w, p->pad_w, p->dil_w);
    int64_t npix = p->n * Ho * Wo, K = npoints(p);
    double *off = (double *)malloc(sizeof(double) * (size_t)(npix * p->groups * K * 2));
    double *mask = (double *)malloc(sizeof(double) * (size_t)(npix * p->groups * K));
    ref_linear(npix, cgd, p->groups * K * 2, guide, w_off, b_off, off);
    ref_linear(npix, cgd, p->groups * K, guide, w_mask, b_mask, mask);
    ref_forward(p, x, off, mask, y);
    free(off);
    free(mask);
}

/* The core followed by the output_proj linear layer w_out (C, C), b_out (C)
 * (b_out may be NULL): out is (N, Ho, Wo, C). */
void ref_forward_proj(const ref_problem *p, const double *x, const double *off, const double *mask,
                      const double *w_out, const double *b_out, double *out)
{
    int64_t Ho = ref_out_size(p->h, p->kh, p->stride_h, p->pad_h, p->dil_h);
    int64_t Wo = ref_out_size(p->w, p->kw, p->stride_w, p->pad_w, p->dil_w);
    int64_t npix = p->n * Ho * Wo;
    double *y = (double *)malloc(sizeof(double) * (size_t)(npix * p->c));
    ref_forward(p, x, off, mask, y);
    ref_linear(npix, p->c, p->c, y, w_out, b_out, out);
    free(y);
}
