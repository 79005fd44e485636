// cbr_launch.h -- host-side plan and launch functions of the CBR kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cbr_common.h"

namespace cbr {

enum ConvEpilogue { EPI_STATS = 0, EPI_BIAS_RELU = 1, EPI_PLAIN = 2 };

// Tile plan of the implicit-GEMM convolution: BM output pixels x BN output channels
// per workgroup.  The plan is a pure function of the geometry, so workspace sizing and
// launches always agree.
struct ConvPlan {
    int bm, bn;
    bool vec;     // input channels a multiple of 8: 16-byte gathers
    int tiles_m, tiles_n;
};
ConvPlan conv_plan(const ConvGeom &g);

// Column sums of a [B][2][K] fp32 partial array: stage 1 folds the B rows into
// colsum_groups(B) <= 64 fp64 rows pp[G][2][K] (fixed order); finalize kernels then
// sum those G rows per channel.
constexpr int COLSUM_MAX_GROUPS = 64;
int colsum_groups(int B);
hipError_t launch_colsum(const float *part, int B, int K, double *pp, hipStream_t st);

// Blocks of the BN-backward reduction over M rows of K channels.
int bnbwd_blocks(int M, int K);

// Split factor of the weight-gradient reduction over output pixels.
struct WgradPlan {
    int bm, bn;       // tile over (K output channels) x (R*S*C)
    int tiles_m, tiles_n, splits;
    int rows_per_split;   // output pixels per split (multiple of the pixel step)
};
WgradPlan wgrad_plan(int M, int K, int Kg);

hipError_t launch_conv_fprop(const ConvGeom &g, int epi, const uint16_t *x, const uint16_t *w,
                             const float *bias, uint16_t *out, float *partials, hipStream_t st);

hipError_t launch_stats_finalize(int tiles_m, int K, long M, const float *partials, double *pp,
                                 const float *gamma, const float *beta, const float *rm_in,
                                 const float *rv_in, float eps, float momentum, float *scale,
                                 float *shift, float *saved_mean, float *saved_invstd,
                                 float *rm_out, float *rv_out, hipStream_t st);

hipError_t launch_bn_apply_relu_mask(long M, int K, const uint16_t *z, const float *scale,
                                     const float *shift, uint16_t *y, uint8_t *mask, hipStream_t st);

hipError_t launch_bn_fold(int K, int Kg, const uint16_t *w, const float *bias, const float *gamma,
                          const float *beta, const float *rm, const float *rv, float eps,
                          uint16_t *w_fold, float *b_fold, hipStream_t st);

hipError_t launch_bn_backward(long M, int K, const uint16_t *dy, const uint8_t *mask,
                              const uint16_t *z, const float *gamma, const float *saved_mean,
                              const float *saved_invstd, float *part, double *pp, float *coef,
                              float *dgamma, float *dbeta, uint16_t *dz, hipStream_t st);

hipError_t launch_flip_weights(int K, int R, int S, int C, const uint16_t *w, uint16_t *wt,
                               hipStream_t st);

hipError_t launch_conv_wgrad(const ConvGeom &g, const uint16_t *dz, const uint16_t *x,
                             float *part, float *dw, hipStream_t st);

}  // namespace cbr
