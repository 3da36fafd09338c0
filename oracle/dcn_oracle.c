/*
 * dcn_oracle.c -- plain, slow CPU oracle for the DCNv3/DCNv4 deformable
 * sampling core.  TEST INFRASTRUCTURE ONLY: nothing on the product path may
 * link, load or call this file.  It shares no code, header or table with the
 * HIP library; the two agree only through the mathematics below.
 *
 * Pages cited (title, site):
 *   [FB]  "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读"
 *         (running InternImage-G without CUDA kernels: the DCNv3 pure-PyTorch
 *         fallback read line by line), trdm.cn
 *   [V4]  "DCNv4高效实践指南：掌握可变形卷积的3倍速度提升技术"
 *         (DCNv4 practice guide), seekfood.cn
 *   [A100] "告别DCNv3的卡顿：实测DCNv4在A100上3倍提速…" (DCNv4 measured 3x
 *         faster on A100), framerc.cn
 *
 * What is computed (the plain definition of the core, [FB] section 4,
 * steps 1-5, rewritten from normalised grid coordinates into pixel units of
 * the unpadded map):
 *
 *   out[n,ho,wo,g*Cg+c] = sum_{i<K, j<K} m[n,ho,wo,g,p] * B(in[n,:,:,g*Cg+c], x_p, y_p),
 *   p   = i*K + j        (i: kernel column / x, j: kernel row / y)
 *   x_p = (wo*s - pad + c0) + alpha * ((i*d - c0) + dx[n,ho,wo,g,p])
 *   y_p = (ho*s - pad + c0) + alpha * ((j*d - c0) + dy[n,ho,wo,g,p])
 *   c0  = floor(d*(K-1)/2)
 *   B   = bilinear read with every pixel outside [0,H)x[0,W) equal to zero
 *   m   = softmax over the P points of each (pixel, group) when softmax != 0
 *         ([FB] section 3 item 3: DCNv3 normalises the modulation mask with a
 *         softmax), the raw mask otherwise ([V4] core architecture section and
 *         [A100] section 1: DCNv4 drops the softmax).
 *
 * Step 1 of [FB] pads the map with zeros; reading the padded map with the
 * zero padding mode of the bilinear sampler is the same as reading the
 * unpadded map with zero outside it, so no padded copy is formed here.
 * Step 2 forms each output pixel's reference point (pixel centre of the
 * padded map) plus the dilation grid scaled by offset_scale; step 3 adds
 * offset*offset_scale; step 4 samples bilinearly (zeros outside, pixel
 * centres at integer+0.5 in normalised units, which is integer pixel
 * coordinates here); step 5 weights by the mask and sums over P.
 *
 * Coordinate precision: coord_mode 0 forms x_p, y_p in binary64 (the exact
 * real-number definition up to one rounding).  coord_mode 1 forms them in
 * binary32 in the fixed order the library documents:
 *     b = fmaf(alpha, (float)(i*d - c0), (float)(wo*s - pad + c0));
 *     x = fmaf(alpha, dx, b)
 * (b is exact when alpha is 1) so that both sides land on the same floor()
 * branch; everything after the coordinates (weights, products, sums,
 * softmax) is binary64 in both modes.
 *
 * Build with -ffp-contract=off so the compiler fuses nothing it was not told
 * to (the two fmaf calls above are explicit).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops below use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Output extent of a convolution-shaped sampling grid ([FB] section 4 step 1
 * takes H_out/W_out from the offset tensor; a stride of 2 halves it). */
int oracle_out_size(int in, int K, int stride, int pad, int dil)
{
    if (in <= 0 || K <= 0 || stride <= 0 || pad < 0 || dil <= 0) return 0;
    long span = (long)dil * (K - 1) + 1;
    long num = (long)in + 2L * pad - span;
    if (num < 0) return 0;
    return (int)(num / stride + 1);
}

/* One sampling coordinate along one axis. */
static double coord(int o, int s, int pad, int c0, int tap, int d, double alpha,
                    double delta, int coord_mode)
{
    if (coord_mode == 1) {
        float b = fmaf((float)alpha, (float)(tap * d - c0), (float)(o * s - pad + c0));
        return (double)fmaf((float)alpha, (float)delta, b);
    }
    return (double)(o * s - pad + c0) + alpha * ((double)(tap * d - c0) + delta);
}

/* Index of tap (i, j) among the P points of a (pixel, group): p = i*K + j,
 * or, with remove_center (DCNv4 option, odd K), the same order with the
 * centre tap left out (P = K*K - 1).  Returns -1 for the removed tap. */
static int point_index(int i, int j, int K, int remove_center)
{
    int p = i * K + j, centre = (K * K - 1) / 2;
    if (!remove_center) return p;
    if (p == centre) return -1;
    return p < centre ? p : p - 1;
}

/* Mask values of one (pixel, group): raw, or softmax over P in binary64. */
static void modulation(const double* logits, int P, int softmax, double* m)
{
    if (!softmax) {
        for (int p = 0; p < P; ++p) m[p] = logits[p];
        return;
    }
    double mx = logits[0];
    for (int p = 1; p < P; ++p)
        if (logits[p] > mx) mx = logits[p];
    double sum = 0.0;
    for (int p = 0; p < P; ++p) { m[p] = exp(logits[p] - mx); sum += m[p]; }
    for (int p = 0; p < P; ++p) m[p] /= sum;
}

/* A sample contributes only if some corner lies on the map: x in (-1, W),
 * y in (-1, H).  NaN coordinates fail every comparison and are skipped. */
static int sample_touches_map(double x, double y, int H, int W)
{
    return x > -1.0 && x < (double)W && y > -1.0 && y < (double)H;
}

/*
 * Forward.  input (N,H,W,G*Cg); offset (N,Ho,Wo,G,P,2) holding (dx,dy);
 * mask (N,Ho,Wo,G,P); out (N,Ho,Wo,G*Cg).  absum (same shape as out, may be
 * NULL) receives sum |m_p * w_corner * f| over the terms of each output, the
 * scale of the rounding error any fp evaluation of the sum can make.
 * Returns 0, or -1 on invalid sizes.
 */
int oracle_forward(const double* input, const double* offset, const double* mask,
                   double* out, double* absum,
                   int N, int H, int W, int G, int Cg, int K, int stride, int pad,
                   int dil, double alpha, int softmax, int coord_mode, int remove_center)
{
    int Ho = oracle_out_size(H, K, stride, pad, dil);
    int Wo = oracle_out_size(W, K, stride, pad, dil);
    if (N <= 0 || G <= 0 || Cg <= 0 || Ho <= 0 || Wo <= 0) return -1;
    if (remove_center && (K % 2 == 0 || K < 3)) return -1;
    const int P = K * K - (remove_center ? 1 : 0), C = G * Cg, c0 = dil * (K - 1) / 2;

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n)
    for (int ho = 0; ho < Ho; ++ho) {
        double* m = (double*)malloc(sizeof(double) * P);
        for (int wo = 0; wo < Wo; ++wo)
        for (int g = 0; g < G; ++g) {
            long pix = ((long)n * Ho + ho) * Wo + wo;
            const double* off = offset + (pix * G + g) * P * 2;
            modulation(mask + (pix * G + g) * P, P, softmax, m);
            double* o = out + pix * C + (long)g * Cg;
            double* a = absum ? absum + pix * C + (long)g * Cg : NULL;
            for (int c = 0; c < Cg; ++c) { o[c] = 0.0; if (a) a[c] = 0.0; }

            for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j) {
                int p = point_index(i, j, K, remove_center);
                if (p < 0) continue;
                double x = coord(wo, stride, pad, c0, i, dil, alpha, off[2 * p], coord_mode);
                double y = coord(ho, stride, pad, c0, j, dil, alpha, off[2 * p + 1], coord_mode);
                if (!sample_touches_map(x, y, H, W)) continue;
                double fx = floor(x), fy = floor(y);
                int x0 = (int)fx, y0 = (int)fy;
                double lx = x - fx, ly = y - fy;
                for (int cy = 0; cy < 2; ++cy)
                for (int cx = 0; cx < 2; ++cx) {
                    int yy = y0 + cy, xx = x0 + cx;
                    if (yy < 0 || yy >= H || xx < 0 || xx >= W) continue;
                    double w = (cy ? ly : 1.0 - ly) * (cx ? lx : 1.0 - lx);
                    const double* f = input + (((long)n * H + yy) * W + xx) * C + (long)g * Cg;
                    for (int c = 0; c < Cg; ++c) {
                        double term = m[p] * w * f[c];
                        o[c] += term;
                        if (a) a[c] += fabs(term);
                    }
                }
            }
        }
        free(m);
    }
    return 0;
}

/*
 * Backward: the analytic gradients of the forward above with respect to
 * input, offset and mask, given grad_out (N,Ho,Wo,G*Cg).  The pages print no
 * gradient formulas; these are the derivatives of the piecewise-bilinear
 * definition, one-sided from the right where the floor() jumps.
 *
 *   v_p[c]       = sum_corners w * f                      (bilinear sample)
 *   grad_in      += m_p * w * g[c]        at every valid corner
 *   gm_p          = sum_c g[c] * v_p[c]
 *   grad_mask_p   = gm_p                                   (raw mask)
 *                 = m_p * (gm_p - sum_q m_q gm_q)          (softmax logits)
 *   grad_dx_p     = alpha * m_p * sum_c g[c] * dv_p[c]/dx
 *   dv/dx = (1-ly)(f01 - f00) + ly(f11 - f10),  dv/dy = (1-lx)(f10 - f00) + lx(f11 - f01)
 * with off-map corners reading zero and skipped samples contributing nothing.
 *
 * grad_input is overwritten (zeroed first).  The *_abs arrays (may be NULL)
 * receive the sums of |elementary terms| for each gradient entry and gi_cnt
 * the number of terms added into each grad_input entry.  Parallel over n.
 */
int oracle_backward(const double* input, const double* offset, const double* mask,
                    const double* grad_out,
                    double* grad_input, double* grad_offset, double* grad_mask,
                    double* gi_abs, double* gi_cnt, double* goff_abs, double* gmask_abs,
                    int N, int H, int W, int G, int Cg, int K, int stride, int pad,
                    int dil, double alpha, int softmax, int coord_mode, int remove_center)
{
    int Ho = oracle_out_size(H, K, stride, pad, dil);
    int Wo = oracle_out_size(W, K, stride, pad, dil);
    if (N <= 0 || G <= 0 || Cg <= 0 || Ho <= 0 || Wo <= 0) return -1;
    if (remove_center && (K % 2 == 0 || K < 3)) return -1;
    const int P = K * K - (remove_center ? 1 : 0), C = G * Cg, c0 = dil * (K - 1) / 2;
    long in_elems = (long)N * H * W * C;
    memset(grad_input, 0, sizeof(double) * in_elems);
    if (gi_abs) memset(gi_abs, 0, sizeof(double) * in_elems);
    if (gi_cnt) memset(gi_cnt, 0, sizeof(double) * in_elems);

#pragma omp parallel for schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        double* m = (double*)malloc(sizeof(double) * P);
        double* gm = (double*)malloc(sizeof(double) * P);
        double* gm_abs = (double*)malloc(sizeof(double) * P);
        for (int ho = 0; ho < Ho; ++ho)
        for (int wo = 0; wo < Wo; ++wo)
        for (int g = 0; g < G; ++g) {
            long pix = ((long)n * Ho + ho) * Wo + wo;
            long pg = pix * G + g;
            const double* off = offset + pg * P * 2;
            const double* go = grad_out + pix * C + (long)g * Cg;
            modulation(mask + pg * P, P, softmax, m);

            for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j) {
                int p = point_index(i, j, K, remove_center);
                if (p < 0) continue;
                double gdx = 0.0, gdy = 0.0, adx = 0.0, ady = 0.0;
                gm[p] = 0.0; gm_abs[p] = 0.0;
                double x = coord(wo, stride, pad, c0, i, dil, alpha, off[2 * p], coord_mode);
                double y = coord(ho, stride, pad, c0, j, dil, alpha, off[2 * p + 1], coord_mode);
                const int touches = sample_touches_map(x, y, H, W);
                if (touches) {
                    double fx = floor(x), fy = floor(y);
                    int x0 = (int)fx, y0 = (int)fy;
                    double lx = x - fx, ly = y - fy;
                    for (int cy = 0; cy < 2; ++cy)
                    for (int cx = 0; cx < 2; ++cx) {
                        int yy = y0 + cy, xx = x0 + cx;
                        if (yy < 0 || yy >= H || xx < 0 || xx >= W) continue;
                        double wy = cy ? ly : 1.0 - ly, wx = cx ? lx : 1.0 - lx;
                        double w = wy * wx;
                        /* d(w)/dx and d(w)/dy of this corner's weight */
                        double dwx = (cx ? 1.0 : -1.0) * wy;
                        double dwy = (cy ? 1.0 : -1.0) * wx;
                        long base = (((long)n * H + yy) * W + xx) * C + (long)g * Cg;
                        const double* f = input + base;
                        for (int c = 0; c < Cg; ++c) {
                            double gf = go[c] * f[c];
                            gm[p] += w * gf;        gm_abs[p] += fabs(w * gf);
                            gdx += dwx * gf;        adx += fabs(dwx * gf);
                            gdy += dwy * gf;        ady += fabs(dwy * gf);
                            double t = m[p] * w * go[c];
                            grad_input[base + c] += t;
                            if (gi_abs) gi_abs[base + c] += fabs(t);
                            if (gi_cnt) gi_cnt[base + c] += 1.0;
                        }
                    }
                }
                /* A skipped sample adds nothing to the output whatever its
                 * offsets are (nearby offsets are skipped too), so its offset
                 * gradient is exactly zero -- also for an Inf or NaN mask
                 * value, which the skipped sample never multiplies. */
                double* god = grad_offset + pg * P * 2;
                god[2 * p] = touches ? alpha * m[p] * gdx : 0.0;
                god[2 * p + 1] = touches ? alpha * m[p] * gdy : 0.0;
                if (goff_abs) {
                    goff_abs[pg * P * 2 + 2 * p] = touches ? fabs(alpha * m[p]) * adx : 0.0;
                    goff_abs[pg * P * 2 + 2 * p + 1] = touches ? fabs(alpha * m[p]) * ady : 0.0;
                }
            }
            double* gmk = grad_mask + pg * P;
            if (!softmax) {
                for (int p = 0; p < P; ++p) {
                    gmk[p] = gm[p];
                    if (gmask_abs) gmask_abs[pg * P + p] = gm_abs[p];
                }
            } else {
                double dot = 0.0, dot_abs = 0.0;
                for (int q = 0; q < P; ++q) { dot += m[q] * gm[q]; dot_abs += m[q] * gm_abs[q]; }
                for (int p = 0; p < P; ++p) {
                    gmk[p] = m[p] * (gm[p] - dot);
                    if (gmask_abs) gmask_abs[pg * P + p] = m[p] * (gm_abs[p] + dot_abs);
                }
            }
        }
        free(m); free(gm); free(gm_abs);
    }
    return 0;
}
