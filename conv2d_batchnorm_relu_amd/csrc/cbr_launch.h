// cbr_launch.h -- host-side plan and launch functions of the CBR kernels (internal).
//
// Every launch function takes an optional pair of events (e0, e1): when either is set,
// the first kernel of the stage is launched with hipExtLaunchKernelGGL recording e0 at
// its start and the last kernel records e1 at its end, so the events bracket exactly
// the stage's kernels (no extra marker packets in the stream).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "cbr_common.h"

namespace cbr {

// Conv epilogues: statistics (training), bias + ReLU (folded-BN inference, and the plain
// Conv2D + ReLU), plain (data gradient), bias without activation.  A NULL bias reads as
// zeros.
enum ConvEpilogue { EPI_STATS = 0, EPI_BIAS_RELU = 1, EPI_PLAIN = 2, EPI_BIAS = 3 };

// Arguments of the BN finalize: per-channel inputs and outputs (float [K] each).
struct BnFinalizeArgs {
    const float *gamma, *beta, *rm_in, *rv_in;
    float eps, momentum;
    double M;                     // samples per channel, N*P*Q
    float *scale, *shift;         // eq_scale, eq_bias of the apply pass
    float *saved_mean, *saved_invstd, *rm_out, *rv_out;
};

// Launches kernel k, recording e0 at its start and e1 at its end when either is set.
template <typename Kern, typename... Args>
inline hipError_t launch(Kern k, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st, hipEvent_t e0,
                         hipEvent_t e1, Args... args)
{
    if (e0 || e1)
        hipExtLaunchKernelGGL(k, grid, block, shmem, st, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(k, grid, block, shmem, st, args...);
    return hipGetLastError();
}

// Raises func's dynamic-LDS limit to at least `bytes` on the current device, calling
// hipFuncSetAttribute only the first time a (function, device) pair needs more (the
// attribute is per device).  Thread-safe.
hipError_t raise_lds_limit(const void *func, int bytes);

// Kernel plans.  Each convolution stage of a call -- the training forward's conv, the
// inference / conv + bias conv, the data gradient's conv and the weight gradient -- runs
// one of these kernels and tile shapes.  resolve_plan picks it per geometry: a tuning
// override if one is set, else the compiled-in table the offline tuner writes, else the
// default rule; every path returns a plan that is eligible for the geometry.  The choice
// is a pure function of (geometry, stage, override), so workspace sizing and launches
// agree.
enum Stage { STAGE_TRAIN = 0, STAGE_INFER = 1, STAGE_DGRAD = 2, STAGE_WGRAD = 3, STAGE_BWD = 4, NSTAGES = 5 };
enum Plan {
    PLAN_DEFAULT = 0,
    PLAN_PERSIST3X3 = 1,    // persistent 3x3 / 64-channel conv + statistics (training only)
    PLAN_FIRST_LAYER = 2,   // 3-channel stride-2 first-layer conv + statistics (training only)
    PLAN_IG_224X256 = 3,    // persistent large-tile conv, 224 x 256 chunks (K % 256 == 0)
    PLAN_IG_448X128 = 4,    // persistent large-tile conv, 448 x 128 chunks (K % 128 == 0)
    PLAN_GEN_128X128 = 5,   // generic implicit-GEMM conv, 128 x 128 tiles
    PLAN_GEN_128X64 = 6,    // generic implicit-GEMM conv, 128 x 64 tiles
    PLAN_WG_TR = 7,         // weight gradient with transposed LDS reads (C % 128, K % 256)
    PLAN_WG_GEN = 8,        // generic weight gradient
    PLAN_BWD_SERIAL = 9,    // backward: weight gradient, then data gradient, one stream
    PLAN_BWD_OVERLAP = 10,  // backward: weight gradient on a second stream beside the data gradient
    PLAN_BWD_FUSED = 11,    // backward: no dz tensor; both gradients form dz while staging (K <= 256, C % 8 == 0)
    PLAN_WG_TR_WIDE = 12,   // weight gradient with transposed LDS reads, 256 x 256 tiles (C % 256, K % 256)
    NPLANS = 13
};
// g is always the layer's geometry (cbr_shape); for STAGE_DGRAD the plan runs, and is
// checked on, the data gradient's convolution dgrad_geom(g).
bool plan_eligible(const ConvGeom &g, int stage, int plan);
int resolve_plan(const ConvGeom &g, int stage);
int default_plan(const ConvGeom &g, int stage);
ConvGeom dgrad_geom(const ConvGeom &g);
const char *plan_name(int plan);
bool set_plan_override(int stage, int plan);

// Tile plan of the generic implicit-GEMM convolution: BM output pixels x BN output
// channels per workgroup.
struct ConvPlan {
    int bm, bn;
    bool vec;     // input channels a multiple of 8: 16-byte gathers
    int tiles_m, tiles_n;
};
ConvPlan conv_plan(const ConvGeom &g, int plan);

// Persistent 3x3 / stride 1 / pad 1, 64 -> 64 channel convolution + channel statistics.
constexpr int HALO_MAX_GRID = 256;                        // one workgroup per MI355X CU
constexpr int HALO_MAX_LDS = 160 * 1024;                  // the whole LDS of a CU
bool halo_eligible(const ConvGeom &g);
int halo_grid(const ConvGeom &g);
size_t halo_lds_bytes(const ConvGeom &g);
hipError_t launch_conv3x3_c64_stats(const ConvGeom &g, const uint16_t *x, const uint16_t *w, uint16_t *z,
                                    float *partials, hipStream_t st, hipEvent_t e0, hipEvent_t e1);

// First-layer conv (3 input channels, stride 2, 64 output channels) + channel statistics:
// persistent, one workgroup per CU over contiguous ranges of 128-pixel steps, MFMA and
// epilogue waves specialised; pixels widened to 4 channels in an LDS ring of input rows,
// the filter to [64][R][8][4] in LDS by each workgroup; one statistics row per workgroup
// (c3s2_grid rows).
bool c3s2_eligible(const ConvGeom &g);
int c3s2_grid(const ConvGeom &g);
size_t c3s2_lds_bytes(const ConvGeom &g);
hipError_t launch_conv_c3s2_stats(const ConvGeom &g, const uint16_t *x, const uint16_t *w, uint16_t *z,
                                  float *partials, hipStream_t st, hipEvent_t e0, hipEvent_t e1);

// Rows of per-channel partial statistics the training forward produces.  The partials
// area holds R rows of [2][K] fp32 (each channel's mean over the row's output pixels,
// then its M2 = sum of squared deviations from that mean), followed by R fp32 pixel
// counts; a row with count 0 holds zeros.
int train_partial_rows(const ConvGeom &g, int plan);

// Blocks of the BN-backward reduction over M rows of K channels.
int bnbwd_blocks(int M, int K);

// Split factor of the weight-gradient reduction over output pixels.
struct WgradPlan {
    bool tr;          // transposed-read kernel (C % bn == 0, K % 256 == 0)
    int bm, bn;       // tile over (K output channels) x (R*S*C)
    int tiles_m, tiles_n, splits;
    int rows_per_split;   // output pixels per split (multiple of the pixel step)
};
bool wgrad_tr_eligible(const ConvGeom &g);
bool wgrad_tr_wide_eligible(const ConvGeom &g);
WgradPlan wgrad_plan(const ConvGeom &g, int plan);

// Persistent large-tile implicit-GEMM conv (C % 32 == 0, K a multiple of the chunk's
// channels): at most 256 workgroups, each over a contiguous range of output pixels; with
// EPI_STATS one partial row per pixel chunk.  plan: PLAN_IG_224X256 or PLAN_IG_448X128.
bool igemm_eligible(const ConvGeom &g, int epi, int plan);
int igemm_partial_rows(const ConvGeom &g, int plan);
hipError_t launch_conv_igemm(const ConvGeom &g, int epi, int plan, const uint16_t *x, const uint16_t *w,
                             const float *bias, uint16_t *out, float *partials, hipStream_t st, hipEvent_t e0,
                             hipEvent_t e1);

// A forward convolution with epilogue epi on the large-tile or the generic kernel, as
// plan says (PLAN_IG_* or PLAN_GEN_*).
hipError_t launch_conv_fprop(const ConvGeom &g, int epi, int plan, const uint16_t *x, const uint16_t *w,
                             const float *bias, uint16_t *out, float *partials, hipStream_t st,
                             hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

hipError_t launch_stats_finalize(int rows, int K, const float *partials, const BnFinalizeArgs &fin, hipStream_t st,
                                 hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

hipError_t launch_bn_apply_relu_mask(long M, int K, const uint16_t *z, const float *scale,
                                     const float *shift, uint16_t *y, uint8_t *mask, hipStream_t st,
                                     hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

hipError_t launch_bn_fold(int K, int Kg, const uint16_t *w, const float *bias, const float *gamma,
                          const float *beta, const float *rm, const float *rv, float eps,
                          uint16_t *w_fold, float *b_fold, hipStream_t st,
                          hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// The masked BN backward: reduce, finalize (dgamma, dbeta and the [5][K] coefficient
// table of bnbwd_dz8 in coef), then dz unless dz is NULL (the fused gradients form it).
hipError_t launch_bn_backward(long M, int K, const uint16_t *dy, const uint8_t *mask,
                              const uint16_t *z, const float *gamma, const float *saved_mean,
                              const float *saved_invstd, float *part, float *coef,
                              float *dgamma, float *dbeta, uint16_t *dz, hipStream_t st,
                              hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// The fused gradients (PLAN_BWD_FUSED): the generic weight-gradient kernel and the
// generic conv of the data gradient with dz formed on load from dy, z, mask and the
// [5][K] coefficient table of bnbwd_dz8 (the data gradient's table needs K <= 256).
hipError_t launch_conv_wgrad_fused(const ConvGeom &g, const uint16_t *dy, const uint16_t *z, const uint8_t *mask,
                                   const float *bnc, const uint16_t *x, float *part, size_t part_bytes, float *dw,
                                   hipStream_t st, hipEvent_t e0, hipEvent_t e1);
hipError_t launch_conv_dgrad_fused(const ConvGeom &d, const uint16_t *dy, const uint16_t *z, const uint8_t *mask,
                                   const float *bnc, const uint16_t *wt, uint16_t *dx, hipStream_t st, hipEvent_t e0,
                                   hipEvent_t e1);

hipError_t launch_flip_weights(int K, int R, int S, int C, const uint16_t *w, uint16_t *wt,
                               hipStream_t st, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// part: the split partials, part_bytes long; a plan whose splits need more is refused
// (hipErrorInvalidValue) before any launch.
hipError_t launch_conv_wgrad(const ConvGeom &g, int plan, const uint16_t *dz, const uint16_t *x,
                             float *part, size_t part_bytes, float *dw, hipStream_t st,
                             hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

}  // namespace cbr
