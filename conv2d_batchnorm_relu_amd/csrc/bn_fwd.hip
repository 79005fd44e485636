// bn_fwd.hip -- batch-norm finalize, normalise + ReLU + packed mask, and the BN fold.
#include "cbr_launch.h"
#include "cbr_reduce.h"

namespace cbr {
namespace {

constexpr int NT = 256;

// The BN finalize (bn_finalize_channel) over the R partial rows ([R][2][K] per-row means
// and M2, then the [R] row counts).  Block b owns channels 4b..4b+3.
template <int NTB>
__global__ __launch_bounds__(NTB) void stats_finalize_kernel(const float *__restrict__ rows, int R, int K,
                                                            BnFinalizeArgs f)
{
    __shared__ double red[8 * NTB / 64];
    const int k0 = 4 * blockIdx.x;
    double mean[4], m2[4];
    chan_combine4<NTB>(rows, rows + (size_t)R * 2 * K, R, K, f.M, k0, mean, m2, red);
    if (threadIdx.x < 4) {
        // thread e finalizes channel k0 + e (constant indices: the arrays stay in registers)
        const int e = threadIdx.x;
        const double me = e == 0 ? mean[0] : e == 1 ? mean[1] : e == 2 ? mean[2] : mean[3];
        const double qe = e == 0 ? m2[0] : e == 1 ? m2[1] : e == 2 ? m2[2] : m2[3];
        bn_finalize_channel(f, k0 + e, me, qe);
    }
}

// Normalise + ReLU + mask (CBR page, section 4.3): u = z*eq_scale + eq_bias, y = max(u, 0),
// mask bit = (u > 0), one pass over z.  Each thread handles UNROLL 16-byte chunks of
// eight channels; chunk c covers elements 8c..8c+7 of the NHWC linear order, so its
// eight mask bits are byte c of the little-endian packed mask.  With FIXEDK the chunk's
// channel group is the same for every chunk a thread visits (256 % (K/8) == 0), so the
// per-channel coefficients are loaded once.  Two chunks per thread (3136 blocks on the
// headline layer): 30.7 us against 32.2 with four and 36-37 with one.
constexpr int APPLY_UNROLL = 2;

template <bool FIXEDK>
__global__ __launch_bounds__(NT) void bn_apply_relu_mask_kernel(const u32x4 *__restrict__ z,
                                                                const float *__restrict__ scale,
                                                                const float *__restrict__ shift,
                                                                u32x4 *__restrict__ y,
                                                                uint8_t *__restrict__ mask, int chunks, int cpr)
{
    const int base = blockIdx.x * NT * APPLY_UNROLL + threadIdx.x;
    float sc[8], sf[8];
    if constexpr (FIXEDK) {
        const int k0 = (threadIdx.x % cpr) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sc[e] = scale[k0 + e];
            sf[e] = shift[k0 + e];
        }
    }
    u32x4 v[APPLY_UNROLL];
#pragma unroll
    for (int u = 0; u < APPLY_UNROLL; ++u) {
        const int c = base + u * NT;
        v[u] = c < chunks ? z[c] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < APPLY_UNROLL; ++u) {
        const int c = base + u * NT;
        if (c >= chunks) break;
        if constexpr (!FIXEDK) {
            const int k0 = (c % cpr) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sc[e] = scale[k0 + e];
                sf[e] = shift[k0 + e];
            }
        }
        uint32_t bits = 0;
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float u0 = fmaf(bf16_lo(v[u][h]), sc[2 * h], sf[2 * h]);
            const float u1 = fmaf(bf16_hi(v[u][h]), sc[2 * h + 1], sf[2 * h + 1]);
            const bool p0 = u0 > 0.f, p1 = u1 > 0.f;
            bits |= (uint32_t)p0 << (2 * h);
            bits |= (uint32_t)p1 << (2 * h + 1);
            o[h] = pack_bf16x2(p0 ? u0 : 0.f, p1 ? u1 : 0.f);
        }
        y[c] = u32x4{o[0], o[1], o[2], o[3]};
        mask[c] = (uint8_t)bits;
        if (c == chunks - 1)   // zero the unused bytes of the last mask word
            for (int t = chunks; t < ((chunks + 3) & ~3); ++t) mask[t] = 0;
    }
}

// The BN fold (CBR page, section 2; BatchNorm CUDA page, section 4.4):
// s_k = gamma_k / sqrt(run_var_k + eps), w_fold = bf16(w * s_k),
// b_fold_k = (b_k - run_mean_k) * s_k + beta_k.
__global__ __launch_bounds__(NT) void bn_fold_kernel(const uint16_t *__restrict__ w, const float *__restrict__ bias,
                                                     const float *__restrict__ gamma, const float *__restrict__ beta,
                                                     const float *__restrict__ rm, const float *__restrict__ rv,
                                                     float eps, int K, int Kg, uint16_t *__restrict__ wf,
                                                     float *__restrict__ bf)
{
    // block k folds output channel k: s_k once, then its Kg filter values (8 per 16-byte
    // chunk when the rows are whole chunks; the row's first chunks are loaded before the
    // scale's arithmetic, so the two latencies overlap)
    const int k = blockIdx.x;
    const uint16_t *wk = w + (size_t)k * Kg;
    uint16_t *wfk = wf + (size_t)k * Kg;
    const bool vec = Kg % 8 == 0;
    const int i0 = threadIdx.x;
    u32x4 first = u32x4{0u, 0u, 0u, 0u};
    if (vec && 8 * i0 < Kg) first = *(const u32x4 *)(wk + 8 * i0);
    const double sd = (double)gamma[k] / sqrt((double)rv[k] + (double)eps);
    const float sf = (float)sd;
    if (vec) {
        auto scale8 = [&](u32x4 v) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack_bf16x2(bf16_bits_to_f32(v[e] & 0xffffu) * sf, bf16_bits_to_f32(v[e] >> 16) * sf);
            return o;
        };
        if (8 * i0 < Kg) *(u32x4 *)(wfk + 8 * i0) = scale8(first);
        for (int i = i0 + NT; 8 * i < Kg; i += NT) *(u32x4 *)(wfk + 8 * i) = scale8(*(const u32x4 *)(wk + 8 * i));
    } else {
        for (int i = threadIdx.x; i < Kg; i += NT) wfk[i] = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(wk[i]) * sf);
    }
    if (threadIdx.x == 0) {
        const double b = bias ? (double)bias[k] : 0.0;
        bf[k] = (float)((b - (double)rm[k]) * sd + (double)beta[k]);
    }
}

}  // namespace

int train_partial_rows(const ConvGeom &g, int plan)
{
    switch (plan) {
    case PLAN_PERSIST3X3: return halo_grid(g);
    case PLAN_FIRST_LAYER: return c3s2_grid(g);
    case PLAN_IG_224X256:
    case PLAN_IG_448X128: return igemm_partial_rows(g, plan);
    default: return conv_plan(g, plan).tiles_m;
    }
}

hipError_t launch_stats_finalize(int rows, int K, const float *partials, const BnFinalizeArgs &fin, hipStream_t st,
                                 hipEvent_t e0, hipEvent_t e1)
{
    if (rows <= COLSUM_SMALL_R)
        return launch(stats_finalize_kernel<COLSUM_NT_SMALL>, dim3(K / 4), dim3(COLSUM_NT_SMALL), 0, st, e0, e1, partials,
                      rows, K, fin);
    return launch(stats_finalize_kernel<COLSUM_NT_LARGE>, dim3(K / 4), dim3(COLSUM_NT_LARGE), 0, st, e0, e1, partials,
                  rows, K, fin);
}

hipError_t launch_bn_apply_relu_mask(long M, int K, const uint16_t *z, const float *scale,
                                     const float *shift, uint16_t *y, uint8_t *mask, hipStream_t st,
                                     hipEvent_t e0, hipEvent_t e1)
{
    const int chunks = (int)(M * K / 8);
    const int cpr = K / 8;
    const int blocks = (chunks + NT * APPLY_UNROLL - 1) / (NT * APPLY_UNROLL);
    if (NT % cpr == 0)
        return launch(bn_apply_relu_mask_kernel<true>, dim3(blocks), dim3(NT), 0, st, e0, e1, (const u32x4 *)z,
                      scale, shift, (u32x4 *)y, mask, chunks, cpr);
    return launch(bn_apply_relu_mask_kernel<false>, dim3(blocks), dim3(NT), 0, st, e0, e1, (const u32x4 *)z, scale,
                  shift, (u32x4 *)y, mask, chunks, cpr);
}

hipError_t launch_bn_fold(int K, int Kg, const uint16_t *w, const float *bias, const float *gamma,
                          const float *beta, const float *rm, const float *rv, float eps,
                          uint16_t *w_fold, float *b_fold, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    return launch(bn_fold_kernel, dim3(K), dim3(NT), 0, st, e0, e1, w, bias, gamma, beta, rm, rv, eps, K, Kg, w_fold,
                  b_fold);
}

}  // namespace cbr
