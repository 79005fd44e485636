/*
 * cbr_oracle.c -- plain fp64 CPU oracle for the fused Conv2D -> BatchNorm -> ReLU
 * (CBR) operator: training forward, folded-BN inference, backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the HIP
 * library and its Python binding) never links, imports or calls it, and shares no
 * code, header, table or helper with it.
 *
 * Every function is the plain definition of what it computes, written as a direct
 * loop nest in double precision.  No blocking, no fusion, no reordering beyond what
 * the definition states; OpenMP only splits the outermost independent loops.
 *
 * Sources (the pages are cited by title and section):
 *   [CBR]  Tech-Renaissance blog, "(20) CBR fused operator: Conv + BatchNorm + ReLU"
 *   [BN]   "CUDA implementation of batch normalization (BatchNorm)" (dpshk.com)
 *   [TL]   "TileLang operator-fusion case: Conv2D+ReLU"
 *   [BURN] "Burn custom CubeCL kernel in practice"
 *
 * Layouts: activations NHWC, filters KRSC ([CBR] section 8, layout constraint),
 * conv output NPQK; all arrays dense row-major, fp64.  Masks are one byte per
 * element (0 or 1): the plain form of the predicate, not the GPU's packed form.
 *
 * Readings where the pages are silent (each listed in the design doc):
 *   - convolution is cross-correlation (no filter flip), dilation 1, groups 1,
 *     symmetric zero padding, output size floor((in + 2*pad - k)/stride) + 1;
 *   - the batch variance is the biased one (divide by M = N*P*Q), [CBR] 4.2;
 *   - momentum weights the new batch statistic, [CBR] 4.2 and [BN] 2.4;
 *   - eps sits inside the square root, [CBR] section 2 and 4.2;
 *   - ReLU mask is the strict predicate u > 0, [CBR] 4.3 (CMP_GT).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX4(a, b, c, d, B, C, D) ((((size_t)(a) * (B) + (b)) * (C) + (c)) * (D) + (d))

/* Output spatial size of a strided, zero-padded cross-correlation. */
int cbro_out_size(int in, int pad, int ksize, int stride)
{
    return (in + 2 * pad - ksize) / stride + 1;
}

/*
 * z[n,p,q,k] = bias[k] + sum_{r,s,c} x[n, p*sh - ph + r, q*sw - pw + s, c] * w[k,r,s,c]
 * with out-of-range input rows/columns read as zero.
 * [CBR] section 2 (y = conv(x, W, b)); [TL] basic convolution (NHWC data, the
 * reduction runs over kernel rows, kernel columns and input channels).
 * bias may be NULL (no bias).
 */
void cbro_conv2d(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                 const double *x, const double *w, const double *bias, double *z)
{
    const int P = cbro_out_size(H, ph, R, sh), Q = cbro_out_size(W, pw, S, sw);
#pragma omp parallel for collapse(2) schedule(static)
    for (int n = 0; n < N; ++n)
        for (int p = 0; p < P; ++p)
            for (int q = 0; q < Q; ++q)
                for (int k = 0; k < K; ++k) {
                    double acc = bias ? bias[k] : 0.0;
                    for (int r = 0; r < R; ++r) {
                        const int h = p * sh - ph + r;
                        if (h < 0 || h >= H) continue;
                        for (int s = 0; s < S; ++s) {
                            const int v = q * sw - pw + s;
                            if (v < 0 || v >= W) continue;
                            const double *xp = x + IDX4(n, h, v, 0, H, W, C);
                            const double *wp = w + IDX4(k, r, s, 0, R, S, C);
                            for (int c = 0; c < C; ++c) acc += xp[c] * wp[c];
                        }
                    }
                    z[IDX4(n, p, q, k, P, Q, K)] = acc;
                }
}

/*
 * The same definition evaluated only at the listed linear NPQK indices
 * (for checking sampled outputs of very large problems).
 */
void cbro_conv2d_at(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                    const double *x, const double *w, const double *bias,
                    long count, const int64_t *idx, double *out)
{
    const int P = cbro_out_size(H, ph, R, sh), Q = cbro_out_size(W, pw, S, sw);
    (void)N;
#pragma omp parallel for schedule(static)
    for (long i = 0; i < count; ++i) {
        int64_t t = idx[i];
        const int k = (int)(t % K); t /= K;
        const int q = (int)(t % Q); t /= Q;
        const int p = (int)(t % P); t /= P;
        const int n = (int)t;
        double acc = bias ? bias[k] : 0.0;
        for (int r = 0; r < R; ++r) {
            const int h = p * sh - ph + r;
            if (h < 0 || h >= H) continue;
            for (int s = 0; s < S; ++s) {
                const int v = q * sw - pw + s;
                if (v < 0 || v >= W) continue;
                for (int c = 0; c < C; ++c)
                    acc += x[IDX4(n, h, v, c, H, W, C)] * w[IDX4(k, r, s, c, R, S, C)];
            }
        }
        out[i] = acc;
    }
}

/*
 * Conv2D + bias with an optional ReLU, no batch normalisation:
 *   y = conv(x, w) + bias                  (relu == 0; [CBR] section 2, y = conv(x, W, b))
 *   y = max(conv(x, w) + bias, 0)          (relu != 0; [TL] fused ReLU section)
 * bias may be NULL (no bias).
 */
void cbro_conv2d_bias_act(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                          const double *x, const double *w, const double *bias, int relu, double *y)
{
    const int P = cbro_out_size(H, ph, R, sh), Q = cbro_out_size(W, pw, S, sw);
    cbro_conv2d(N, H, W, C, K, R, S, sh, sw, ph, pw, x, w, bias, y);
    if (relu) {
        const size_t total = (size_t)N * P * Q * K;
        for (size_t i = 0; i < total; ++i) y[i] = y[i] > 0.0 ? y[i] : 0.0;
    }
}

/*
 * Per-channel batch statistics of z viewed as [M][K]:
 *   mean_k = (1/M) sum_m z[m,k],   var_k = (1/M) sum_m (z[m,k] - mean_k)^2.
 * [BN] 2.1 (mean and variance over N x H x W per channel); [CBR] 4.2 defines
 * var = E[z^2] - mean^2 with N_ac = N*H*W samples, equal to this two-pass form in
 * exact arithmetic; the two-pass form is used here because it does not cancel.
 */
void cbro_batch_stats(long M, int K, const double *z, double *mean, double *var)
{
    for (int k = 0; k < K; ++k) { mean[k] = 0.0; var[k] = 0.0; }
    for (long m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) mean[k] += z[(size_t)m * K + k];
    for (int k = 0; k < K; ++k) mean[k] /= (double)M;
    for (long m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) {
            const double d = z[(size_t)m * K + k] - mean[k];
            var[k] += d * d;
        }
    for (int k = 0; k < K; ++k) var[k] /= (double)M;
}

/*
 * Training-mode forward ([CBR] sections 2, 4.1-4.3; [BN] 2.1 and 2.4):
 *   z            = conv(x, w)                       (no conv bias: the training
 *                                                    operator's inputs carry none)
 *   mean, var    = batch statistics of z per output channel (biased variance)
 *   invstd       = 1 / sqrt(var + eps)
 *   u            = gamma * (z - mean) * invstd + beta
 *   y            = max(u, 0),  mask = (u > 0)
 *   run_mean_out = (1 - momentum) * run_mean_in + momentum * mean
 *   run_var_out  = (1 - momentum) * run_var_in  + momentum * var
 * saved_mean = mean and saved_invstd = invstd are kept for the backward pass.
 * batch_var receives var (it is what the running update consumes).
 */
void cbro_forward_train(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                        const double *x, const double *w, const double *gamma, const double *beta,
                        const double *run_mean_in, const double *run_var_in, double eps, double momentum,
                        double *z, double *y, uint8_t *mask, double *batch_var,
                        double *saved_mean, double *saved_invstd,
                        double *run_mean_out, double *run_var_out)
{
    const int P = cbro_out_size(H, ph, R, sh), Q = cbro_out_size(W, pw, S, sw);
    const long M = (long)N * P * Q;
    cbro_conv2d(N, H, W, C, K, R, S, sh, sw, ph, pw, x, w, NULL, z);
    cbro_batch_stats(M, K, z, saved_mean, batch_var);
    for (int k = 0; k < K; ++k) saved_invstd[k] = 1.0 / sqrt(batch_var[k] + eps);
#pragma omp parallel for schedule(static)
    for (long m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) {
            const size_t i = (size_t)m * K + k;
            const double u = gamma[k] * (z[i] - saved_mean[k]) * saved_invstd[k] + beta[k];
            mask[i] = (uint8_t)(u > 0.0);
            y[i] = u > 0.0 ? u : 0.0;
        }
    for (int k = 0; k < K; ++k) {
        run_mean_out[k] = (1.0 - momentum) * run_mean_in[k] + momentum * saved_mean[k];
        run_var_out[k] = (1.0 - momentum) * run_var_in[k] + momentum * batch_var[k];
    }
}

/*
 * Inference forward by definition, with the running statistics in place of the
 * batch ones ([CBR] section 2; [BN] 2.4):
 *   u = gamma * (conv(x, w) + b - run_mean) / sqrt(run_var + eps) + beta,  y = max(u, 0).
 * bias may be NULL (no conv bias).  This does NOT use the folded weights: the fold is
 * checked against this function, not the other way round.
 */
void cbro_forward_infer(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                        const double *x, const double *w, const double *bias,
                        const double *gamma, const double *beta,
                        const double *run_mean, const double *run_var, double eps,
                        double *z_scratch, double *y)
{
    const int P = cbro_out_size(H, ph, R, sh), Q = cbro_out_size(W, pw, S, sw);
    const long M = (long)N * P * Q;
    cbro_conv2d(N, H, W, C, K, R, S, sh, sw, ph, pw, x, w, bias, z_scratch);
#pragma omp parallel for schedule(static)
    for (long m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) {
            const size_t i = (size_t)m * K + k;
            const double u = gamma[k] * (z_scratch[i] - run_mean[k]) / sqrt(run_var[k] + eps) + beta[k];
            y[i] = u > 0.0 ? u : 0.0;
        }
}

/*
 * The BN-into-conv fold ([CBR] section 2; [BN] 4.4):
 *   w_fold[k,r,s,c] = w[k,r,s,c] * gamma[k] / sqrt(run_var[k] + eps)
 *   b_fold[k]       = (b[k] - run_mean[k]) * gamma[k] / sqrt(run_var[k] + eps) + beta[k]
 * bias may be NULL (read as zero).
 */
void cbro_fold(int K, int R, int S, int C, const double *w, const double *bias,
               const double *gamma, const double *beta, const double *run_mean,
               const double *run_var, double eps, double *w_fold, double *b_fold)
{
    for (int k = 0; k < K; ++k) {
        const double scale = gamma[k] / sqrt(run_var[k] + eps);
        const size_t per = (size_t)R * S * C;
        for (size_t j = 0; j < per; ++j) w_fold[(size_t)k * per + j] = w[(size_t)k * per + j] * scale;
        b_fold[k] = ((bias ? bias[k] : 0.0) - run_mean[k]) * scale + beta[k];
    }
}

/*
 * ReLU-masked BN backward for z viewed as [M][K] ([CBR] section 5.1: dY is multiplied
 * by the forward mask first; [BN] 3.1, the s1/s2/count form):
 *   g      = dy * mask
 *   xhat   = (z - saved_mean) * saved_invstd
 *   dbeta  = sum_m g,   dgamma = sum_m g * xhat
 *   dz     = gamma * saved_invstd * (g - dbeta/M - xhat * dgamma/M)
 * xhat is recomputed from the stored conv output and the saved statistics.
 */
void cbro_bn_backward(long M, int K, const double *dy, const uint8_t *mask, const double *z,
                      const double *gamma, const double *saved_mean, const double *saved_invstd,
                      double *dz, double *dgamma, double *dbeta)
{
    for (int k = 0; k < K; ++k) { dgamma[k] = 0.0; dbeta[k] = 0.0; }
    for (long m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) {
            const size_t i = (size_t)m * K + k;
            const double g = mask[i] ? dy[i] : 0.0;
            const double xhat = (z[i] - saved_mean[k]) * saved_invstd[k];
            dbeta[k] += g;
            dgamma[k] += g * xhat;
        }
#pragma omp parallel for schedule(static)
    for (long m = 0; m < M; ++m)
        for (int k = 0; k < K; ++k) {
            const size_t i = (size_t)m * K + k;
            const double g = mask[i] ? dy[i] : 0.0;
            const double xhat = (z[i] - saved_mean[k]) * saved_invstd[k];
            dz[i] = gamma[k] * saved_invstd[k] * (g - dbeta[k] / (double)M - xhat * dgamma[k] / (double)M);
        }
}

/*
 * Data gradient of the convolution: the adjoint of cbro_conv2d in x.  Every output
 * term x[n,h,v,c]*w[k,r,s,c] that fed z[n,p,q,k] sends dz[n,p,q,k]*w[k,r,s,c] back to
 * x[n,h,v,c] ([CBR] section 5.2, DGrad from dL/d(conv_out) and W; [BURN] step 4,
 * grad_lhs = grad * rhs^T for the GEMM form).  Any stride.
 */
void cbro_conv2d_dgrad(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                       const double *dz, const double *w, double *dx)
{
    const int P = cbro_out_size(H, ph, R, sh), Q = cbro_out_size(W, pw, S, sw);
    memset(dx, 0, sizeof(double) * (size_t)N * H * W * C);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
        for (int p = 0; p < P; ++p)
            for (int q = 0; q < Q; ++q)
                for (int k = 0; k < K; ++k) {
                    const double g = dz[IDX4(n, p, q, k, P, Q, K)];
                    for (int r = 0; r < R; ++r) {
                        const int h = p * sh - ph + r;
                        if (h < 0 || h >= H) continue;
                        for (int s = 0; s < S; ++s) {
                            const int v = q * sw - pw + s;
                            if (v < 0 || v >= W) continue;
                            double *dxp = dx + IDX4(n, h, v, 0, H, W, C);
                            const double *wp = w + IDX4(k, r, s, 0, R, S, C);
                            for (int c = 0; c < C; ++c) dxp[c] += g * wp[c];
                        }
                    }
                }
}

/*
 * Weight gradient of the convolution:
 *   dw[k,r,s,c] = sum_{n,p,q} dz[n,p,q,k] * x[n, p*sh - ph + r, q*sw - pw + s, c]
 * ([CBR] section 5.2, WGrad from dL/d(conv_out) and X; [BURN] step 4,
 * grad_rhs = lhs^T * grad for the GEMM form).
 */
void cbro_conv2d_wgrad(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                       const double *dz, const double *x, double *dw)
{
    const int P = cbro_out_size(H, ph, R, sh), Q = cbro_out_size(W, pw, S, sw);
#pragma omp parallel for schedule(static)
    for (int k = 0; k < K; ++k) {
        double *dwk = dw + (size_t)k * R * S * C;
        for (size_t j = 0; j < (size_t)R * S * C; ++j) dwk[j] = 0.0;
        for (int n = 0; n < N; ++n)
            for (int p = 0; p < P; ++p)
                for (int q = 0; q < Q; ++q) {
                    const double g = dz[IDX4(n, p, q, k, P, Q, K)];
                    for (int r = 0; r < R; ++r) {
                        const int h = p * sh - ph + r;
                        if (h < 0 || h >= H) continue;
                        for (int s = 0; s < S; ++s) {
                            const int v = q * sw - pw + s;
                            if (v < 0 || v >= W) continue;
                            const double *xp = x + IDX4(n, h, v, 0, H, W, C);
                            double *dwp = dwk + ((size_t)r * S + s) * C;
                            for (int c = 0; c < C; ++c) dwp[c] += g * xp[c];
                        }
                    }
                }
    }
}

/*
 * Whole CBR backward ([CBR] section 5: masked BN backward, then WGrad, then DGrad;
 * the first-layer form of 5.3 skips DGrad, requested here by dx == NULL).
 * Inputs are the forward's saved state: x, w, the conv output z, the ReLU mask and
 * the saved batch statistics, plus gamma and the upstream gradient dy.
 */
void cbro_backward(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                   const double *x, const double *w, const double *z, const uint8_t *mask,
                   const double *dy, const double *gamma, const double *saved_mean,
                   const double *saved_invstd,
                   double *dz, double *dgamma, double *dbeta, double *dw, double *dx)
{
    const int P = cbro_out_size(H, ph, R, sh), Q = cbro_out_size(W, pw, S, sw);
    const long M = (long)N * P * Q;
    cbro_bn_backward(M, K, dy, mask, z, gamma, saved_mean, saved_invstd, dz, dgamma, dbeta);
    cbro_conv2d_wgrad(N, H, W, C, K, R, S, sh, sw, ph, pw, dz, x, dw);
    if (dx) cbro_conv2d_dgrad(N, H, W, C, K, R, S, sh, sw, ph, pw, dz, w, dx);
}

/* Number of OpenMP threads the oracle runs with (for reporting). */
int cbro_num_threads(void)
{
    int t = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        t = omp_get_num_threads();
    }
#endif
    return t;
}

/* Sets the number of OpenMP threads later calls use (n >= 1); timing only, the results
 * do not depend on it (every output element is computed by one thread, in a fixed order). */
void cbro_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
