// bn_bwd.hip -- ReLU-masked batch-norm backward (CBR page, section 5.1; BatchNorm CUDA
// page, sections 3.1-3.3).  Two-stage form of the BatchNorm page's section 3.2:
//   reduce:   per block, s1 = sum g and s2 = sum g*xhat over a range of pixels, with
//             g = dy * mask and xhat = (z - mean) * invstd recomputed from stored z;
//   finalize: dbeta = s1, dgamma = s2 (fp64 over the block partials, fixed order);
//   apply:    dz = gamma*invstd*(g - dbeta/M - xhat*dgamma/M), written as bf16.
// g is never written to memory.
#include "cbr_launch.h"
#include "cbr_reduce.h"

namespace cbr {
namespace {

constexpr int NT = 256;
constexpr int ROW_UNROLL = 4;

__global__ __launch_bounds__(NT) void bnbwd_reduce_kernel(const u32x4 *__restrict__ dy,
                                                          const uint8_t *__restrict__ mask,
                                                          const u32x4 *__restrict__ z,
                                                          const float *__restrict__ mean,
                                                          const float *__restrict__ invstd, int M, int K,
                                                          int rows_per_block, float *__restrict__ part)
{
    __shared__ float red[2][NT * 8];
    const int cpr = K / 8, rpp = NT / cpr;
    const int tid = threadIdx.x, cc = tid % cpr, ro = tid / cpr;
    const int m0 = blockIdx.x * rows_per_block, m1 = min(M, m0 + rows_per_block);
    float s1[8], s2[8], mu[8], is[8];
    const int k0 = cc * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s1[e] = 0.f;
        s2[e] = 0.f;
        mu[e] = mean[k0 + e];
        is[e] = invstd[k0 + e];
    }
    if (ro < rpp) {
        for (int mb = m0 + ro; mb < m1; mb += rpp * ROW_UNROLL) {
            u32x4 zv[ROW_UNROLL], dv[ROW_UNROLL];
            uint32_t mk[ROW_UNROLL];
#pragma unroll
            for (int u = 0; u < ROW_UNROLL; ++u) {
                const int m = mb + u * rpp;
                const bool ok = m < m1;
                const size_t c = (size_t)m * cpr + cc;
                zv[u] = ok ? z[c] : u32x4{0, 0, 0, 0};
                dv[u] = ok ? dy[c] : u32x4{0, 0, 0, 0};
                mk[u] = ok ? mask[c] : 0u;
            }
#pragma unroll
            for (int u = 0; u < ROW_UNROLL; ++u)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float g0 = ((mk[u] >> (2 * h)) & 1u) ? bf16_lo(dv[u][h]) : 0.f;
                    const float g1 = ((mk[u] >> (2 * h + 1)) & 1u) ? bf16_hi(dv[u][h]) : 0.f;
                    const float x0 = (bf16_lo(zv[u][h]) - mu[2 * h]) * is[2 * h];
                    const float x1 = (bf16_hi(zv[u][h]) - mu[2 * h + 1]) * is[2 * h + 1];
                    s1[2 * h] += g0;
                    s1[2 * h + 1] += g1;
                    s2[2 * h] = fmaf(g0, x0, s2[2 * h]);
                    s2[2 * h + 1] = fmaf(g1, x1, s2[2 * h + 1]);
                }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            red[0][ro * K + k0 + e] = s1[e];
            red[1][ro * K + k0 + e] = s2[e];
        }
    }
    __syncthreads();
    for (int k = tid; k < K; k += NT) {
        float a = 0.f, b = 0.f;
        for (int r = 0; r < rpp; ++r) {
            a += red[0][r * K + k];
            b += red[1][r * K + k];
        }
        part[(size_t)blockIdx.x * 2 * K + k] = a;
        part[(size_t)blockIdx.x * 2 * K + K + k] = b;
    }
}

// dbeta = s1, dgamma = s2 (fp64 over the partial rows, fixed order); the coefficient
// table of bnbwd_dz8, [5][K]: mean, invstd, ca = gamma*invstd, cb = dbeta/M,
// cg = dgamma/M.  Block b owns channels 4b..4b+3.
template <int NTB>
__global__ __launch_bounds__(NTB) void bnbwd_finalize_kernel(const float *__restrict__ rows, int R, int K, double M,
                                                            const float *__restrict__ gamma,
                                                            const float *__restrict__ mean,
                                                            const float *__restrict__ invstd,
                                                            float *__restrict__ coef, float *__restrict__ dgamma,
                                                            float *__restrict__ dbeta)
{
    __shared__ double red[8 * NTB / 64];
    const int k0 = 4 * blockIdx.x;
    double s[8];
    colsum_pair4<NTB>(rows, R, K, k0, s, red);
    if (threadIdx.x < 4) {
        const int e = threadIdx.x, k = k0 + e;
        const double s1 = e == 0 ? s[0] : e == 1 ? s[1] : e == 2 ? s[2] : s[3];
        const double s2 = e == 0 ? s[4] : e == 1 ? s[5] : e == 2 ? s[6] : s[7];
        dbeta[k] = (float)s1;
        dgamma[k] = (float)s2;
        coef[k] = mean[k];
        coef[K + k] = invstd[k];
        coef[2 * K + k] = gamma[k] * invstd[k];
        coef[3 * K + k] = (float)(s1 / M);
        coef[4 * K + k] = (float)(s2 / M);
    }
}

constexpr int APPLY_UNROLL = 4;

template <bool FIXEDK>
__global__ __launch_bounds__(NT) void bnbwd_apply_kernel(const u32x4 *__restrict__ dy,
                                                         const uint8_t *__restrict__ mask,
                                                         const u32x4 *__restrict__ z,
                                                         const float *__restrict__ coef, int K,
                                                         u32x4 *__restrict__ dz, int chunks, int cpr)
{
    const int base = blockIdx.x * NT * APPLY_UNROLL + threadIdx.x;
    float mu[8], is[8], ca[8], cb[8], cg[8];
    auto load_coef = [&](int k0) { bnbwd_coef8(coef, K, k0, mu, is, ca, cb, cg); };
    if constexpr (FIXEDK) load_coef((threadIdx.x % cpr) * 8);
    u32x4 zv[APPLY_UNROLL], dv[APPLY_UNROLL];
    uint32_t mk[APPLY_UNROLL];
#pragma unroll
    for (int u = 0; u < APPLY_UNROLL; ++u) {
        const int c = base + u * NT;
        const bool ok = c < chunks;
        zv[u] = ok ? z[c] : u32x4{0, 0, 0, 0};
        dv[u] = ok ? dy[c] : u32x4{0, 0, 0, 0};
        mk[u] = ok ? mask[c] : 0u;
    }
#pragma unroll
    for (int u = 0; u < APPLY_UNROLL; ++u) {
        const int c = base + u * NT;
        if (c >= chunks) break;
        if constexpr (!FIXEDK) load_coef((c % cpr) * 8);
        dz[c] = bnbwd_dz8(dv[u], zv[u], mk[u], mu, is, ca, cb, cg);
    }
}

}  // namespace

int bnbwd_blocks(int M, int K)
{
    const int rpp = NT / (K / 8);
    const int want = (M + rpp * ROW_UNROLL * 4 - 1) / (rpp * ROW_UNROLL * 4);
    return std::max(1, std::min(1024, want));
}

hipError_t launch_bn_backward(long M, int K, const uint16_t *dy, const uint8_t *mask,
                              const uint16_t *z, const float *gamma, const float *saved_mean,
                              const float *saved_invstd, float *part, float *coef,
                              float *dgamma, float *dbeta, uint16_t *dz, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    const int B = bnbwd_blocks((int)M, K);
    const int rpp = NT / (K / 8);
    int rows = (int)((M + B - 1) / B);
    rows = (rows + rpp - 1) / rpp * rpp;
    const int Bn = (int)((M + rows - 1) / rows);
    hipError_t e = launch(bnbwd_reduce_kernel, dim3(Bn), dim3(NT), 0, st, e0, nullptr, (const u32x4 *)dy, mask,
                          (const u32x4 *)z, saved_mean, saved_invstd, (int)M, K, rows, part);
    if (e != hipSuccess) return e;
    if (Bn <= COLSUM_SMALL_R)
        e = launch(bnbwd_finalize_kernel<COLSUM_NT_SMALL>, dim3(K / 4), dim3(COLSUM_NT_SMALL), 0, st, nullptr, dz ? nullptr : e1,
                   (const float *)part, Bn, K, (double)M, gamma, saved_mean, saved_invstd, coef, dgamma, dbeta);
    else
        e = launch(bnbwd_finalize_kernel<COLSUM_NT_LARGE>, dim3(K / 4), dim3(COLSUM_NT_LARGE), 0, st, nullptr, dz ? nullptr : e1,
                   (const float *)part, Bn, K, (double)M, gamma, saved_mean, saved_invstd, coef, dgamma, dbeta);
    if (e != hipSuccess || !dz) return e;
    const int chunks = (int)(M * K / 8);
    const int cpr = K / 8;
    const int blocks = (chunks + NT * APPLY_UNROLL - 1) / (NT * APPLY_UNROLL);
    if (NT % cpr == 0)
        return launch(bnbwd_apply_kernel<true>, dim3(blocks), dim3(NT), 0, st, nullptr, e1, (const u32x4 *)dy, mask,
                      (const u32x4 *)z, (const float *)coef, K, (u32x4 *)dz, chunks, cpr);
    return launch(bnbwd_apply_kernel<false>, dim3(blocks), dim3(NT), 0, st, nullptr, e1, (const u32x4 *)dy, mask,
                  (const u32x4 *)z, (const float *)coef, K, (u32x4 *)dz, chunks, cpr);
}

}  // namespace cbr
