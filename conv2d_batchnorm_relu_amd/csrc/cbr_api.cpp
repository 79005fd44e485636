// cbr_api.cpp -- the C ABI of libcbr.so: argument validation, workspace layout and the
// kernel sequence of each call.  Everything here runs on the host; validation finishes
// before the first HIP call, so a rejected call touches no device state.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/cbr.h"
#include "cbr_launch.h"

using namespace cbr;

namespace {

constexpr size_t ALIGN = 256;

size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

// Validates a shape and fills the forward-convolution geometry.
int make_geom(const cbr_shape *s, ConvGeom *g)
{
    if (!s) return CBR_E_NULL;
    if (s->n <= 0 || s->h <= 0 || s->w <= 0 || s->c <= 0 || s->k <= 0 || s->r <= 0 || s->s <= 0 ||
        s->stride_h < 1 || s->stride_w < 1 || s->pad_h < 0 || s->pad_w < 0)
        return CBR_E_SHAPE;
    const long hp = (long)s->h + 2L * s->pad_h - s->r, wp = (long)s->w + 2L * s->pad_w - s->s;
    if (hp < 0 || wp < 0) return CBR_E_SHAPE;
    const long P = hp / s->stride_h + 1, Q = wp / s->stride_w + 1;
    if (s->k % 8 != 0 || s->k > 2048) return CBR_E_UNSUPPORTED;
    if (s->pad_h >= s->r || s->pad_w >= s->s) return CBR_E_UNSUPPORTED;
    const double lim = 1073741823.0;   // < 2^30 elements: every byte offset fits 31 bits
    if ((double)s->n * s->h * s->w * s->c > lim || (double)s->k * s->r * s->s * s->c > lim ||
        (double)s->n * P * Q * s->k > lim)
        return CBR_E_UNSUPPORTED;
    g->N = s->n; g->H = s->h; g->W = s->w; g->C = s->c;
    g->K = s->k; g->R = s->r; g->S = s->s;
    g->sh = s->stride_h; g->sw = s->stride_w; g->ph = s->pad_h; g->pw = s->pad_w;
    g->P = (int)P; g->Q = (int)Q;
    g->M = (int)(s->n * P * Q);
    g->Kg = s->r * s->s * s->c;
    return CBR_OK;
}

std::mutex g_lds_mu;
std::map<std::pair<const void *, int>, int> g_lds_limit;   // (function, device) -> bytes set

}  // namespace

hipError_t cbr::raise_lds_limit(const void *func, int bytes)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_lds_mu);
    int &have = g_lds_limit[std::make_pair(func, dev)];
    if (have >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) have = bytes;
    return e;
}

// The data gradient as a stride-1 forward convolution of dz with the flipped filter.
ConvGeom cbr::dgrad_geom(const ConvGeom &g)
{
    ConvGeom d;
    d.N = g.N; d.H = g.P; d.W = g.Q; d.C = g.K;
    d.K = g.C; d.R = g.R; d.S = g.S;
    d.sh = 1; d.sw = 1; d.ph = g.R - 1 - g.ph; d.pw = g.S - 1 - g.pw;
    d.P = g.H; d.Q = g.W;
    d.M = g.N * g.H * g.W;
    d.Kg = g.R * g.S * g.K;
    return d;
}

namespace {

struct TrainLayout { size_t partials, scale, shift, total; };
struct InferLayout { size_t wfold, bfold, total; };
struct BwdLayout { size_t dz, part, coef, wpart, wflip, total; };

TrainLayout train_layout(const ConvGeom &g, int plan)
{
    TrainLayout L;
    size_t o = 0;
    L.partials = o; o = align_up(o + sizeof(float) * (2 * g.K + 1) * (size_t)train_partial_rows(g, plan));
    L.scale = o; o = align_up(o + sizeof(float) * g.K);
    L.shift = o; o = align_up(o + sizeof(float) * g.K);
    L.total = o;
    return L;
}

InferLayout infer_layout(const ConvGeom &g)
{
    InferLayout L;
    size_t o = 0;
    L.wfold = o; o = align_up(o + sizeof(uint16_t) * (size_t)g.K * g.Kg);
    L.bfold = o; o = align_up(o + sizeof(float) * g.K);
    L.total = o;
    return L;
}

// Bytes of the weight gradient's split partials for plan wplan (0 when it takes one split).
size_t wgrad_part_bytes(const ConvGeom &g, int wplan)
{
    const WgradPlan wp = wgrad_plan(g, wplan);
    return wp.splits > 1 ? sizeof(float) * (size_t)wp.splits * g.K * g.Kg : 0;
}

// wplan: the weight-gradient stage's plan; the partials also cover the generic weight
// gradient when the backward's schedule may form dz inside the gradients (which always
// runs the generic kernel, whose split count can be larger).
BwdLayout bwd_layout(const ConvGeom &g, int wplan)
{
    BwdLayout L;
    size_t part_bytes = wgrad_part_bytes(g, wplan);
    if (resolve_plan(g, STAGE_BWD) == PLAN_BWD_FUSED) part_bytes = std::max(part_bytes, wgrad_part_bytes(g, PLAN_WG_GEN));
    size_t o = 0;
    L.dz = o; o = align_up(o + sizeof(uint16_t) * (size_t)g.M * g.K);
    L.part = o; o = align_up(o + sizeof(float) * 2 * g.K * (size_t)bnbwd_blocks(g.M, g.K));
    L.coef = o; o = align_up(o + sizeof(float) * 5 * g.K);
    L.wpart = o; o = align_up(o + part_bytes);
    L.wflip = o; o = align_up(o + sizeof(uint16_t) * (size_t)g.K * g.Kg);
    L.total = o;
    return L;
}

// A second stream per device for the weight gradient, which runs beside the data
// gradient (the CBR page runs WGrad on a stream of its own, section 5.2), with the two
// events that fork it from and join it back to the caller's stream.  Created on first
// use with the device current and kept for the life of the process; default priority.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr, flip = nullptr;
    std::mutex mu;   // held from each event record to the wait that consumes it
};
constexpr int MAX_DEVICES = 64;
SideStream g_side[MAX_DEVICES];
std::mutex g_side_mu;

SideStream *side_stream()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream &ss = g_side[dev];
    if (!ss.stream) {
        hipStream_t st = nullptr;
        hipEvent_t a = nullptr, b = nullptr, c = nullptr;
        if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
        if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&c, hipEventDisableTiming) != hipSuccess) {
            if (a) (void)hipEventDestroy(a);
            if (b) (void)hipEventDestroy(b);
            (void)hipStreamDestroy(st);
            return nullptr;
        }
        ss.fork = a;
        ss.join = b;
        ss.flip = c;
        ss.stream = st;
    }
    return &ss;
}

// Makes `waiter` wait for everything enqueued so far on `source`, through event ev.
hipError_t stream_after(hipStream_t waiter, hipStream_t source, hipEvent_t ev)
{
    hipError_t e = hipEventRecord(ev, source);
    if (e == hipSuccess) e = hipStreamWaitEvent(waiter, ev, 0);
    return e;
}

bool ranges_overlap(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

template <typename... T>
bool all_aligned(T... ps) { return (aligned16(ps) && ...); }

template <typename... T>
bool any_null(T... ps) { return ((ps == nullptr) || ...); }

char *ws_at(void *ws, size_t off) { return (char *)ws + off; }

// Profiling event i, or none.
hipEvent_t ev(void *const *events, int i) { return events ? (hipEvent_t)events[i] : nullptr; }

}  // namespace

extern "C" {

const char *cbr_status_str(int status)
{
    switch (status) {
    case CBR_OK: return "CBR_OK";
    case CBR_E_NULL: return "CBR_E_NULL: a required pointer is NULL";
    case CBR_E_SHAPE: return "CBR_E_SHAPE: invalid shape (sizes, stride, padding, empty output, or one output pixel in training)";
    case CBR_E_UNSUPPORTED: return "CBR_E_UNSUPPORTED: shape outside the supported limits";
    case CBR_E_ALIGN: return "CBR_E_ALIGN: a tensor pointer is not 16-byte aligned";
    case CBR_E_WORKSPACE: return "CBR_E_WORKSPACE: workspace missing or too small";
    case CBR_E_HIP: return "CBR_E_HIP: a kernel launch failed";
    case CBR_E_VALUE: return "CBR_E_VALUE: eps or momentum out of range";
    default: return "CBR: unknown status";
    }
}

int cbr_output_hw(const cbr_shape *shape, int32_t *p, int32_t *q)
{
    ConvGeom g;
    const int st = make_geom(shape, &g);
    if (st != CBR_OK) return st;
    if (p) *p = g.P;
    if (q) *q = g.Q;
    return CBR_OK;
}

size_t cbr_mask_words(const cbr_shape *shape)
{
    ConvGeom g;
    if (make_geom(shape, &g) != CBR_OK) return 0;
    return ((size_t)g.M * g.K + 31) / 32;
}

size_t cbr_workspace_bytes(const cbr_shape *shape, int op)
{
    ConvGeom g;
    if (make_geom(shape, &g) != CBR_OK) return 0;
    switch (op) {
    case CBR_OP_TRAIN: return train_layout(g, resolve_plan(g, STAGE_TRAIN)).total;
    case CBR_OP_INFER: return infer_layout(g).total;
    case CBR_OP_BWD: return bwd_layout(g, resolve_plan(g, STAGE_WGRAD)).total;
    default: return 0;
    }
}

int cbr_forward_train_ev(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *gamma,
                         const float *beta, const float *run_mean_in, const float *run_var_in, float eps,
                         float momentum, uint16_t *z, uint16_t *y, uint32_t *relu_mask, float *saved_mean,
                         float *saved_invstd, float *run_mean_out, float *run_var_out, void *workspace,
                         size_t ws_bytes, void *stream, void *const *events)
{
    ConvGeom g;
    int st = make_geom(shape, &g);
    if (st != CBR_OK) return st;
    if (any_null(x, w, gamma, beta, run_mean_in, run_var_in, z, y, relu_mask, saved_mean, saved_invstd,
                 run_mean_out, run_var_out))
        return CBR_E_NULL;
    if (!all_aligned(x, w, gamma, beta, run_mean_in, run_var_in, z, y, relu_mask, saved_mean, saved_invstd,
                     run_mean_out, run_var_out))
        return CBR_E_ALIGN;
    if (g.M < 2) return CBR_E_SHAPE;   // batch statistics need two values per channel
    if (!(eps >= 0.f) || !isfinite(eps) || !(momentum >= 0.f && momentum <= 1.f)) return CBR_E_VALUE;
    const int plan = resolve_plan(g, STAGE_TRAIN);
    const TrainLayout L = train_layout(g, plan);
    if (!workspace || ws_bytes < L.total) return CBR_E_WORKSPACE;
    if (!aligned16(workspace)) return CBR_E_ALIGN;

    hipStream_t s = (hipStream_t)stream;
    float *partials = (float *)ws_at(workspace, L.partials);
    float *scale = (float *)ws_at(workspace, L.scale);
    float *shift = (float *)ws_at(workspace, L.shift);
    const BnFinalizeArgs fin{gamma, beta,  run_mean_in, run_var_in,   eps,          momentum,   (double)g.M,
                             scale, shift, saved_mean,  saved_invstd, run_mean_out, run_var_out};
    // conv + channel sums (CBR page 4.1) -> finalize (4.2) -> apply + ReLU + mask (4.3)
    const hipError_t ec =
        plan == PLAN_PERSIST3X3
            ? launch_conv3x3_c64_stats(g, x, w, z, partials, s, ev(events, 0), ev(events, 1))
        : plan == PLAN_FIRST_LAYER
            ? launch_conv_c3s2_stats(g, x, w, z, partials, s, ev(events, 0), ev(events, 1))
            : launch_conv_fprop(g, EPI_STATS, plan, x, w, nullptr, z, partials, s, ev(events, 0), ev(events, 1));
    if (ec != hipSuccess) return CBR_E_HIP;
    if (launch_stats_finalize(train_partial_rows(g, plan), g.K, partials, fin, s, ev(events, 2), ev(events, 3)) !=
        hipSuccess)
        return CBR_E_HIP;
    if (launch_bn_apply_relu_mask(g.M, g.K, z, scale, shift, y, (uint8_t *)relu_mask, s, ev(events, 4),
                                  ev(events, 5)) != hipSuccess)
        return CBR_E_HIP;
    return CBR_OK;
}

int cbr_forward_train(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *gamma,
                      const float *beta, const float *run_mean_in, const float *run_var_in, float eps,
                      float momentum, uint16_t *z, uint16_t *y, uint32_t *relu_mask, float *saved_mean,
                      float *saved_invstd, float *run_mean_out, float *run_var_out, void *workspace,
                      size_t ws_bytes, void *stream)
{
    return cbr_forward_train_ev(shape, x, w, gamma, beta, run_mean_in, run_var_in, eps, momentum, z, y,
                                relu_mask, saved_mean, saved_invstd, run_mean_out, run_var_out, workspace,
                                ws_bytes, stream, nullptr);
}

int cbr_forward_infer_ev(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *conv_bias,
                         const float *gamma, const float *beta, const float *run_mean, const float *run_var,
                         float eps, uint16_t *y, void *workspace, size_t ws_bytes, void *stream,
                         void *const *events)
{
    ConvGeom g;
    int st = make_geom(shape, &g);
    if (st != CBR_OK) return st;
    if (any_null(x, w, gamma, beta, run_mean, run_var, y)) return CBR_E_NULL;
    if (!all_aligned(x, w, gamma, beta, run_mean, run_var, y) || (conv_bias && !aligned16(conv_bias)))
        return CBR_E_ALIGN;
    if (!(eps >= 0.f) || !isfinite(eps)) return CBR_E_VALUE;
    const InferLayout L = infer_layout(g);
    if (!workspace || ws_bytes < L.total) return CBR_E_WORKSPACE;
    if (!aligned16(workspace)) return CBR_E_ALIGN;

    hipStream_t s = (hipStream_t)stream;
    uint16_t *wf = (uint16_t *)ws_at(workspace, L.wfold);
    float *bf = (float *)ws_at(workspace, L.bfold);
    if (launch_bn_fold(g.K, g.Kg, w, conv_bias, gamma, beta, run_mean, run_var, eps, wf, bf, s, ev(events, 0),
                       ev(events, 1)) != hipSuccess)
        return CBR_E_HIP;
    if (launch_conv_fprop(g, EPI_BIAS_RELU, resolve_plan(g, STAGE_INFER), x, wf, bf, y, nullptr, s, ev(events, 2),
                          ev(events, 3)) != hipSuccess)
        return CBR_E_HIP;
    return CBR_OK;
}

int cbr_forward_infer(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *conv_bias,
                      const float *gamma, const float *beta, const float *run_mean, const float *run_var,
                      float eps, uint16_t *y, void *workspace, size_t ws_bytes, void *stream)
{
    return cbr_forward_infer_ev(shape, x, w, conv_bias, gamma, beta, run_mean, run_var, eps, y, workspace,
                                ws_bytes, stream, nullptr);
}

// Conv2D + bias (+ ReLU) without batch normalisation: one convolution launch with the
// bias (and ReLU) epilogue.
static int conv_bias_act(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias, bool relu,
                         uint16_t *y, void *stream, void *const *events)
{
    ConvGeom g;
    int st = make_geom(shape, &g);
    if (st != CBR_OK) return st;
    if (any_null(x, w, y)) return CBR_E_NULL;
    if (!all_aligned(x, w, y) || (bias && !aligned16(bias))) return CBR_E_ALIGN;
    if (launch_conv_fprop(g, relu ? EPI_BIAS_RELU : EPI_BIAS, resolve_plan(g, STAGE_INFER), x, w, bias, y, nullptr,
                          (hipStream_t)stream, ev(events, 0), ev(events, 1)) != hipSuccess)
        return CBR_E_HIP;
    return CBR_OK;
}

int cbr_conv2d_bias_relu_ev(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias,
                            uint16_t *y, void *stream, void *const *events)
{
    return conv_bias_act(shape, x, w, bias, true, y, stream, events);
}

int cbr_conv2d_bias_relu(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias, uint16_t *y,
                         void *stream)
{
    return conv_bias_act(shape, x, w, bias, true, y, stream, nullptr);
}

int cbr_conv2d_bias_ev(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias, uint16_t *y,
                       void *stream, void *const *events)
{
    return conv_bias_act(shape, x, w, bias, false, y, stream, events);
}

int cbr_conv2d_bias(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const float *bias, uint16_t *y,
                    void *stream)
{
    return conv_bias_act(shape, x, w, bias, false, y, stream, nullptr);
}

int cbr_backward_ev(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const uint16_t *z,
                    const uint32_t *relu_mask, const uint16_t *dy, const float *gamma, const float *saved_mean,
                    const float *saved_invstd, uint16_t *dz, float *dgamma, float *dbeta, float *dw,
                    uint16_t *dx, void *workspace, size_t ws_bytes, void *stream, void *const *events)
{
    ConvGeom g;
    int st = make_geom(shape, &g);
    if (st != CBR_OK) return st;
    if (any_null(x, w, z, relu_mask, dy, gamma, saved_mean, saved_invstd, dgamma, dbeta, dw)) return CBR_E_NULL;
    if (!all_aligned(x, w, z, relu_mask, dy, gamma, saved_mean, saved_invstd, dgamma, dbeta, dw) ||
        (dz && !aligned16(dz)) || (dx && !aligned16(dx)))
        return CBR_E_ALIGN;
    if (g.M < 2) return CBR_E_SHAPE;
    if (dx && (g.sh != 1 || g.sw != 1)) return CBR_E_UNSUPPORTED;
    const int wplan = resolve_plan(g, STAGE_WGRAD);
    const BwdLayout L = bwd_layout(g, wplan);
    if (!workspace || ws_bytes < L.total) return CBR_E_WORKSPACE;
    if (!aligned16(workspace)) return CBR_E_ALIGN;

    hipStream_t s = (hipStream_t)stream;
    const int bplan = resolve_plan(g, STAGE_BWD);
    if (bplan == PLAN_BWD_FUSED && !dz) {
        // No dz tensor: the BN backward stops at its coefficients, and both gradients form
        // dz from dy, z and the mask as they stage their operands (generic kernels; the
        // data gradient after the weight gradient, as dx may alias x).
        float *coef = (float *)ws_at(workspace, L.coef);
        if (launch_bn_backward(g.M, g.K, dy, (const uint8_t *)relu_mask, z, gamma, saved_mean, saved_invstd,
                               (float *)ws_at(workspace, L.part), coef, dgamma, dbeta, nullptr, s, ev(events, 0),
                               ev(events, 1)) != hipSuccess)
            return CBR_E_HIP;
        if (launch_conv_wgrad_fused(g, dy, z, (const uint8_t *)relu_mask, coef, x, (float *)ws_at(workspace, L.wpart),
                                    L.wflip - L.wpart, dw, s, ev(events, 2), ev(events, 3)) != hipSuccess)
            return CBR_E_HIP;
        if (dx) {
            uint16_t *wt = (uint16_t *)ws_at(workspace, L.wflip);
            if (launch_flip_weights(g.K, g.R, g.S, g.C, w, wt, s, ev(events, 4), nullptr) != hipSuccess)
                return CBR_E_HIP;
            const ConvGeom d = dgrad_geom(g);
            if (launch_conv_dgrad_fused(d, dy, z, (const uint8_t *)relu_mask, coef, wt, dx, s, nullptr,
                                        ev(events, 5)) != hipSuccess)
                return CBR_E_HIP;
        } else if (events && (hipEventRecord(ev(events, 4), s) != hipSuccess ||
                              hipEventRecord(ev(events, 5), s) != hipSuccess)) {
            return CBR_E_HIP;
        }
        return CBR_OK;
    }
    uint16_t *dzp = dz ? dz : (uint16_t *)ws_at(workspace, L.dz);
    // The weight gradient runs beside the data gradient on the side stream when the plan
    // says so and dx does not overlap x (the data gradient would overwrite what the
    // weight gradient reads, the in-place hazard of the CBR page's section 5.2);
    // otherwise both run on the caller's stream, weight gradient first.
    const size_t xbytes = (size_t)g.N * g.H * g.W * g.C * 2;
    // The device's side stream (default priority): the data gradient's filter flip, which
    // reads only w, runs on it beside the BN backward; with the overlap plan the weight
    // gradient follows it there, beside the data gradient.  Its lock is held from the
    // first event record to the last wait of this call.
    const bool overlap = dx && bplan == PLAN_BWD_OVERLAP && !ranges_overlap(dx, xbytes, x, xbytes);
    SideStream *ss = dx ? side_stream() : nullptr;
    std::unique_lock<std::mutex> side_lock;
    uint16_t *wt = (uint16_t *)ws_at(workspace, L.wflip);
    if (ss) {
        side_lock = std::unique_lock<std::mutex>(ss->mu);
        // the side stream first waits for the caller's earlier work (w may have just been
        // written on it)
        if (stream_after(ss->stream, s, ss->fork) != hipSuccess) return CBR_E_HIP;
        if (launch_flip_weights(g.K, g.R, g.S, g.C, w, wt, ss->stream, nullptr, nullptr) != hipSuccess)
            return CBR_E_HIP;
        if (hipEventRecord(ss->flip, ss->stream) != hipSuccess) return CBR_E_HIP;
    } else if (dx && launch_flip_weights(g.K, g.R, g.S, g.C, w, wt, s, nullptr, nullptr) != hipSuccess) {
        return CBR_E_HIP;
    }
    // masked BN backward (CBR page 5.1) -> WGrad, DGrad (5.2; DGrad skipped for the first
    // layer, 5.3).
    if (launch_bn_backward(g.M, g.K, dy, (const uint8_t *)relu_mask, z, gamma, saved_mean, saved_invstd,
                           (float *)ws_at(workspace, L.part),
                           (float *)ws_at(workspace, L.coef), dgamma, dbeta, dzp, s, ev(events, 0),
                           ev(events, 1)) != hipSuccess)
        return CBR_E_HIP;
    if (overlap && ss && stream_after(ss->stream, s, ss->fork) != hipSuccess) return CBR_E_HIP;
    const bool wg_side = overlap && ss;
    if (launch_conv_wgrad(g, wplan, dzp, x, (float *)ws_at(workspace, L.wpart), L.wflip - L.wpart, dw,
                          wg_side ? ss->stream : s, ev(events, 2), ev(events, 3)) != hipSuccess)
        return CBR_E_HIP;
    if (wg_side && hipEventRecord(ss->join, ss->stream) != hipSuccess) return CBR_E_HIP;
    if (dx) {
        if (ss && hipStreamWaitEvent(s, ss->flip, 0) != hipSuccess) return CBR_E_HIP;
        const ConvGeom d = dgrad_geom(g);
        // the dgrad stage's events bracket the conv (the flip ran beside the BN backward)
        if (launch_conv_fprop(d, EPI_PLAIN, resolve_plan(g, STAGE_DGRAD), dzp, wt, nullptr, dx, nullptr, s,
                              ev(events, 4), ev(events, 5)) != hipSuccess)
            return CBR_E_HIP;
    } else if (events && (hipEventRecord(ev(events, 4), s) != hipSuccess ||
                          hipEventRecord(ev(events, 5), s) != hipSuccess)) {
        return CBR_E_HIP;
    }
    // the caller's stream continues only once the weight gradient has finished
    if (wg_side && hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return CBR_E_HIP;
    return CBR_OK;
}

int cbr_backward(const cbr_shape *shape, const uint16_t *x, const uint16_t *w, const uint16_t *z,
                 const uint32_t *relu_mask, const uint16_t *dy, const float *gamma, const float *saved_mean,
                 const float *saved_invstd, uint16_t *dz, float *dgamma, float *dbeta, float *dw, uint16_t *dx,
                 void *workspace, size_t ws_bytes, void *stream)
{
    return cbr_backward_ev(shape, x, w, z, relu_mask, dy, gamma, saved_mean, saved_invstd, dz, dgamma, dbeta, dw,
                           dx, workspace, ws_bytes, stream, nullptr);
}

int cbr_plan_of(const cbr_shape *shape, int stage)
{
    ConvGeom g;
    const int st = make_geom(shape, &g);
    if (st != CBR_OK) return -st;
    if (stage < 0 || stage >= NSTAGES) return -CBR_E_VALUE;
    return resolve_plan(g, stage);
}

int cbr_plan_eligible(const cbr_shape *shape, int stage, int plan)
{
    ConvGeom g;
    const int st = make_geom(shape, &g);
    if (st != CBR_OK) return -st;
    if (stage < 0 || stage >= NSTAGES) return -CBR_E_VALUE;
    return plan_eligible(g, stage, plan) ? 1 : 0;
}

const char *cbr_plan_name(int plan) { return plan_name(plan); }

int cbr_set_plan_override(int stage, int plan) { return set_plan_override(stage, plan) ? CBR_OK : CBR_E_VALUE; }

}  // extern "C"
