/*
 * cbr.h -- C ABI of libcbr.so: the fused Conv2D -> BatchNorm -> ReLU (CBR) operator
 * on AMD Instinct MI355X (gfx950), training forward, folded-BN inference and backward.
 *
 * Pages the operations follow (cited by title and section):
 *   [CBR]  Tech-Renaissance blog, "(20) CBR fused operator: Conv + BatchNorm + ReLU"
 *   [BN]   "CUDA implementation of batch normalization (BatchNorm)" (dpshk.com)
 *   [TL]   "TileLang operator-fusion case: Conv2D+ReLU"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts ([CBR] section 8): activations NHWC, filters KRSC (K = output channels),
 * conv outputs N x P x Q x K, all dense.  P = (H + 2*pad_h - R)/stride_h + 1 and
 * Q = (W + 2*pad_w - S)/stride_w + 1 (floor); the convolution is a cross-correlation
 * with zero padding, dilation 1, one group.  M = N*P*Q is the number of output pixels.
 *
 * Types: tensors marked bf16 are bfloat16 bit patterns (uint16_t); statistics,
 * gamma/beta, the weight gradient and conv bias are float32.
 *
 * Pointers: every tensor pointer is a DEVICE pointer, 16-byte aligned, owned by the
 * caller; no call allocates or frees device memory.  The library keeps two things per
 * device for the life of the process: the scratch array of cbr_forward_train_noalloc
 * (module memory, loaded with the library) and, once cbr_backward has run with a dx
 * there, a second stream with three events (created on that first call).  The cbr_shape
 * pointer is a host pointer read during the call only.  `workspace` is caller-owned
 * device scratch of at least cbr_workspace_bytes(shape, op) bytes (256-byte aligned);
 * its contents are undefined between calls and it must not be shared by calls that
 * may run concurrently.  `stream` is a hipStream_t (NULL = the null stream).
 *
 * Execution: each call validates its arguments on the host, then enqueues its
 * kernels on `stream` and returns without synchronising.  Faults during kernel
 * execution surface at the caller's next synchronisation, as HIP reports them.
 * Results are bitwise reproducible run to run (no floating-point atomics).
 *
 * Errors: a non-zero return means nothing was enqueued and no output was written,
 * except CBR_E_HIP, which reports a failed launch (outputs then undefined).  No call
 * aborts or exits the process.
 *
 * Limits (CBR_E_UNSUPPORTED): K % 8 != 0 ([CBR] section 8: output channels a multiple
 * of 8); K > 2048; any tensor with 2^30 elements or more; pad >= filter size;
 * dx requested with a stride other than 1.
 */
#ifndef CBR_H
#define CBR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cbr_shape {
    int32_t n, h, w, c;                     /* input, NHWC                         */
    int32_t k, r, s;                        /* filter, KRSC (k = output channels)  */
    int32_t stride_h, stride_w, pad_h, pad_w;
} cbr_shape;

enum cbr_status {
    CBR_OK = 0,
    CBR_E_NULL = 1,         /* a required pointer is NULL                            */
    CBR_E_SHAPE = 2,        /* non-positive size, stride < 1, negative pad, empty out,
                               or M < 2 in training (no batch variance from one value) */
    CBR_E_UNSUPPORTED = 3,  /* valid but outside the limits listed above             */
    CBR_E_ALIGN = 4,        /* a tensor pointer is not 16-byte aligned               */
    CBR_E_WORKSPACE = 5,    /* workspace NULL or smaller than cbr_workspace_bytes    */
    CBR_E_HIP = 6,          /* a kernel launch failed                                */
    CBR_E_VALUE = 7         /* eps < 0, momentum outside [0,1], or not finite        */
};

enum cbr_op { CBR_OP_TRAIN = 0, CBR_OP_INFER = 1, CBR_OP_BWD = 2 };

/* Human-readable name of a status code (static string, never NULL). */
const char *cbr_status_str(int status);

/* Checks the shape alone; writes P and Q when they are non-NULL.  Returns a status. */
int cbr_output_hw(const cbr_shape *shape, int32_t *p, int32_t *q);

/* Number of uint32 words of the packed ReLU mask: ceil(M*K / 32). */
size_t cbr_mask_words(const cbr_shape *shape);

/* Workspace bytes that op (enum cbr_op) needs for this shape; 0 for an invalid shape.
 * For CBR_OP_BWD the figure includes room for dz, used when the caller passes dz = NULL. */
size_t cbr_workspace_bytes(const cbr_shape *shape, int op);

/*
 * Training-mode forward ([CBR] sections 2 and 4.1-4.3; [BN] 2.1, 2.4):
 *   z        = conv(x, w)                                   bf16 [N,P,Q,K]  (out)
 *   mean_k   = (1/M) sum z,  var_k = (1/M) sum (z - mean_k)^2   (biased; from the
 *              fp32 accumulators, before z is rounded to bf16)
 *   invstd_k = 1/sqrt(var_k + eps)
 *   u        = gamma_k * (z - mean_k) * invstd_k + beta_k  (computed from stored z)
 *   y        = max(u, 0)                                    bf16 [N,P,Q,K]  (out)
 *   relu_mask: bit (i % 32) of word (i / 32) is (u_i > 0) for the NHWC linear index i
 *              of y; cbr_mask_words() words, bits past M*K are zero        (out)
 *   saved_mean = mean, saved_invstd = invstd                   float [K]   (out)
 *   run_mean_out = (1-momentum)*run_mean_in + momentum*mean    float [K]   (out)
 *   run_var_out  = (1-momentum)*run_var_in  + momentum*var     float [K]   (out)
 * x: bf16 NHWC [N,H,W,C]; w: bf16 KRSC [K,R,S,C]; gamma, beta, run_*_in: float [K].
 * Needs M >= 2 (CBR_E_SHAPE otherwise).  u normalises the stored bf16 z with statistics
 * of the unrounded values, so a channel whose batch variance is below the bf16 rounding
 * error of its values (var << (2^-8 |z|)^2, e.g. a constant non-zero channel) gets u
 * dominated by that rounding error.
 * run_mean_out/run_var_out may alias run_mean_in/run_var_in (in-place update); no other
 * output may alias an input.  There is no conv bias: batch normalisation cancels it.
 */
int cbr_forward_train(const cbr_shape *shape,
                      const uint16_t *x, const uint16_t *w,
                      const float *gamma, const float *beta,
                      const float *run_mean_in, const float *run_var_in,
                      float eps, float momentum,
                      uint16_t *z, uint16_t *y, uint32_t *relu_mask,
                      float *saved_mean, float *saved_invstd,
                      float *run_mean_out, float *run_var_out,
                      void *workspace, size_t ws_bytes, void *stream);

/*
 * Folded-BN inference forward ([CBR] sections 2 and 6; [BN] 4.4; [TL] fused ReLU
 * epilogue):
 *   s_k      = gamma_k / sqrt(run_var_k + eps)
 *   w_fold   = w * s_k (per output channel, rounded to bf16),
 *   b_fold_k = (b_k - run_mean_k) * s_k + beta_k   (float)
 *   y        = max(conv(x, w_fold) + b_fold, 0)                   bf16 [N,P,Q,K] (out)
 * conv_bias may be NULL (read as zero).  All other pointers as in training.
 */
int cbr_forward_infer(const cbr_shape *shape,
                      const uint16_t *x, const uint16_t *w, const float *conv_bias,
                      const float *gamma, const float *beta,
                      const float *run_mean, const float *run_var, float eps,
                      uint16_t *y, void *workspace, size_t ws_bytes, void *stream);

/*
 * Backward of the training forward ([CBR] section 5; [BN] 3.1-3.3):
 *   g      = dy * mask                      (never written to memory)
 *   xhat   = (z - saved_mean) * saved_invstd (recomputed from the stored bf16 z)
 *   dbeta  = sum_m g,  dgamma = sum_m g * xhat                       float [K] (out)
 *   dz     = gamma * saved_invstd * (g - dbeta/M - xhat * dgamma/M)  bf16 [N,P,Q,K]
 *   dw[k,r,s,c] = sum_{n,p,q} dz[n,p,q,k] * x[n, p*sh-ph+r, q*sw-pw+s, c]  float KRSC
 *   dx[n,h,v,c] = sum_{k,r,s} dz[n,p,q,k] * w[k,r,s,c] over the (p,q) that read
 *                 x[n,h,v] through tap (r,s)                           bf16 NHWC
 *   dw and dx are computed from the bf16 dz above (as the CBR page's WGrad and DGrad
 *   read dL/d(conv_out) from a half-precision buffer), accumulated in fp32.
 * Needs M >= 2 (CBR_E_SHAPE otherwise).
 * Inputs: x, w, z (bf16), relu_mask, dy (bf16 [N,P,Q,K]), gamma, saved_mean,
 * saved_invstd (float [K]) -- the training forward's inputs and outputs.
 * dz may be NULL (then it lives in the workspace).  dx may be NULL: the first-layer
 * form of [CBR] 5.3, which skips the data gradient.  dx may alias x: the weight
 * gradient finishes reading x before the data gradient writes dx ([CBR] 5.2).
 * A non-NULL dx needs stride 1 in both directions.
 * With a dx, the data gradient's filter flip (it reads only w) runs on a second stream
 * that the library keeps per device, beside the BN backward; when dx does not overlap x
 * the weight gradient may run there too (see CBR_STAGE_BWD).  Both are forked from and
 * joined back to `stream` with events: the call's work is still complete when `stream`
 * reaches its end.  Calls on one device from several host threads serialise their
 * enqueueing around that stream.
 */
int cbr_backward(const cbr_shape *shape,
                 const uint16_t *x, const uint16_t *w, const uint16_t *z,
                 const uint32_t *relu_mask, const uint16_t *dy,
                 const float *gamma, const float *saved_mean, const float *saved_invstd,
                 uint16_t *dz, float *dgamma, float *dbeta, float *dw, uint16_t *dx,
                 void *workspace, size_t ws_bytes, void *stream);

/*
 * The training forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments
 * and results as cbr_forward_train without the workspace: the kernels' scratch is a
 * CBR_NOALLOC_SCRATCH_BYTES array that the library holds on each device from the first
 * call made with that device current until the process ends (its address is looked up
 * then, with hipGetSymbolAddress).  The call itself allocates nothing.
 * Limit: shapes whose cbr_workspace_bytes(shape, CBR_OP_TRAIN) exceeds
 * CBR_NOALLOC_SCRATCH_BYTES return CBR_E_WORKSPACE (the 256 x 56 x 56 x 64 workload needs
 * about 133 KB, the 224 x 224 first layer at N = 64 also about 133 KB).
 * All calls on one device share that device's array: calls that may overlap on one
 * device (different streams, different host threads) race, and must be serialised by
 * the caller.  A call leaves the array's contents undefined; no call depends on them.
 */
#define CBR_NOALLOC_SCRATCH_BYTES (4u << 20)

int cbr_forward_train_noalloc(const cbr_shape *shape,
                              const uint16_t *x, const uint16_t *w,
                              const float *gamma, const float *beta,
                              const float *run_mean_in, const float *run_var_in,
                              float eps, float momentum,
                              uint16_t *z, uint16_t *y, uint32_t *relu_mask,
                              float *saved_mean, float *saved_invstd,
                              float *run_mean_out, float *run_var_out, void *stream);

/*
 * Conv2D + bias + ReLU without batch normalisation ([TL] "fused ReLU" section: the ReLU
 * applied in the convolution's epilogue, before the result leaves the chip):
 *   y = max(conv(x, w) + bias, 0)                                  bf16 [N,P,Q,K] (out)
 * x: bf16 NHWC [N,H,W,C]; w: bf16 KRSC [K,R,S,C]; bias: float [K], may be NULL (read as
 * zero).  No workspace.  Shape limits and errors as for the other calls.
 */
int cbr_conv2d_bias_relu(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias,
                         uint16_t *y, void *stream);

/*
 * Conv2D + bias without activation ([TL] basic convolution with a bias epilogue; the
 * convolution of [CBR] section 2, y = conv(x, W, b)):
 *   y = conv(x, w) + bias                                          bf16 [N,P,Q,K] (out)
 * Arguments as for cbr_conv2d_bias_relu.
 */
int cbr_conv2d_bias(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias,
                    uint16_t *y, void *stream);

/*
 * Kernel plans (tuning interface).  Each convolution stage of a call runs one kernel and
 * tile shape, its "plan", chosen per shape like the per-shape engine choice of [CBR]
 * section 7 (empirical search, winner per shape) and [TL]'s autotuned tile
 * configurations: a compiled-in table of plans measured offline (tune.py), else a
 * default rule.  Stages: CBR_STAGE_TRAIN_CONV (the conv + statistics of
 * cbr_forward_train), CBR_STAGE_INFER_CONV (the conv of cbr_forward_infer and of the
 * conv + bias calls), CBR_STAGE_DGRAD (the data gradient's conv), CBR_STAGE_WGRAD (the
 * weight gradient), CBR_STAGE_BWD (how cbr_backward schedules its gradients).  Plans:
 * 1 persistent 3x3/64-channel conv, 2 first-layer conv, 3 large-tile 224x256,
 * 4 large-tile 448x128, 5 generic 128x128, 6 generic 128x64, 7 weight gradient with
 * transposed reads, 8 generic weight gradient, 9 backward on one stream (weight gradient,
 * then data gradient), 10 backward with the weight gradient on a second stream beside the
 * data gradient ([CBR] section 5.2's WGrad stream; used only when dx does not overlap x,
 * else the call falls back to 9), 11 backward with no dz tensor: both gradients form dz
 * from dy, z and the mask while staging their operands ([CBR] section 5.1 keeps the
 * masked gradient on chip; K <= 256 and C % 8 == 0; used only when dz is NULL, else
 * the call falls back to 9), 12 weight gradient with transposed reads on 256 x 256 tiles
 * (C % 256 == 0 and K % 256 == 0).
 *
 * cbr_plan_of: the plan the stage will run for this layer shape (> 0), or minus a status.
 * cbr_plan_eligible: 1 if the plan can run the stage for this shape, 0 if not, or minus
 *   a status for an invalid shape or stage.
 * cbr_plan_name: a static name of a plan id.
 * cbr_set_plan_override: makes the stage run `plan` wherever it is eligible (plan 0
 *   clears it); process-wide, for the tuner and tests only.  cbr_workspace_bytes follows
 *   the override, so query it after setting one.  CBR_E_VALUE for a bad stage or plan.
 */
enum cbr_stage { CBR_STAGE_TRAIN_CONV = 0, CBR_STAGE_INFER_CONV = 1, CBR_STAGE_DGRAD = 2, CBR_STAGE_WGRAD = 3,
                 CBR_STAGE_BWD = 4 };

int cbr_plan_of(const cbr_shape *shape, int stage);
int cbr_plan_eligible(const cbr_shape *shape, int stage, int plan);
const char *cbr_plan_name(int plan);
int cbr_set_plan_override(int stage, int plan);

/*
 * Timed variants for profiling: identical to the calls above, and in addition record
 * caller-created hipEvent_t handles (passed as void*) at the start of the first kernel
 * and the end of the last kernel of each stage (taken from the kernels' own dispatch
 * timestamps, so no marker packets are added to the stream).  `events` may be NULL
 * (then the call is exactly the untimed one).  Event pairs (start, end):
 *   train:  [0,1] convolution + channel sums, [2,3] statistics finalize,
 *           [4,5] normalise + ReLU + mask                                  (6 events)
 *   infer:  [0,1] fold, [2,3] convolution + bias + ReLU                     (4 events)
 *   bwd:    [0,1] BN backward (reduce, finalize, dz), [2,3] weight gradient,
 *           [4,5] data gradient (recorded back to back when dx is NULL)    (6 events)
 *   conv2d_bias(_relu): [0,1] the convolution                             (2 events)
 */
int cbr_forward_train_ev(const cbr_shape *shape,
                         const uint16_t *x, const uint16_t *w,
                         const float *gamma, const float *beta,
                         const float *run_mean_in, const float *run_var_in,
                         float eps, float momentum,
                         uint16_t *z, uint16_t *y, uint32_t *relu_mask,
                         float *saved_mean, float *saved_invstd,
                         float *run_mean_out, float *run_var_out,
                         void *workspace, size_t ws_bytes, void *stream, void *const *events);

int cbr_forward_infer_ev(const cbr_shape *shape,
                         const uint16_t *x, const uint16_t *w, const float *conv_bias,
                         const float *gamma, const float *beta,
                         const float *run_mean, const float *run_var, float eps,
                         uint16_t *y, void *workspace, size_t ws_bytes, void *stream,
                         void *const *events);

int cbr_backward_ev(const cbr_shape *shape,
                    const uint16_t *x, const uint16_t *w, const uint16_t *z,
                    const uint32_t *relu_mask, const uint16_t *dy,
                    const float *gamma, const float *saved_mean, const float *saved_invstd,
                    uint16_t *dz, float *dgamma, float *dbeta, float *dw, uint16_t *dx,
                    void *workspace, size_t ws_bytes, void *stream, void *const *events);

int cbr_conv2d_bias_relu_ev(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias,
                            uint16_t *y, void *stream, void *const *events);

int cbr_conv2d_bias_ev(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias,
                       uint16_t *y, void *stream, void *const *events);

#ifdef __cplusplus
}
#endif

#endif /* CBR_H */
