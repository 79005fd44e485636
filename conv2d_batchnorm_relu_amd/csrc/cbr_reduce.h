// cbr_reduce.h -- per-channel column sums of a row-major [R][2K] float partials array
// (row r: K sums, then K sums of a second quantity), accumulated in fp64 in a fixed
// order, so results are reproducible bit for bit; and the BN finalize of one channel.
#pragma once

#include "cbr_launch.h"

namespace cbr {

// Threads per block of the column-sum kernels: one wave for up to COLSUM_SMALL_R rows
// (the reduction then needs no LDS and no barrier), four waves for more rows.
constexpr int COLSUM_NT_SMALL = 64, COLSUM_NT_LARGE = 256, COLSUM_SMALL_R = 1024;
// Rows a thread loads in one batch (all in flight together).
constexpr int COLSUM_UN = 8;

// Sum of a[0..NV-1] over the NTB threads of a block, in fp64 and a fixed order: a
// butterfly over the 64 lanes of each wave (lane shuffles; the two operands of every
// addition are the same at both lanes, so all lanes hold identical sums), then, for
// several waves, the wave sums in wave order through LDS (red: 8 * NTB / 64 doubles).
// On return every thread holds the block sums in a[].
template <int NTB, int NV>
__device__ inline void block_sum(double (&a)[NV], double *red)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < NV; ++e) a[e] += __shfl_xor(a[e], off);
    if constexpr (NTB > 64) {
        static_assert(NV <= 8, "red holds 8 values per wave");
        const int w = threadIdx.x >> 6;
        __syncthreads();   // red is free (a previous use has been read)
        if ((threadIdx.x & 63) == 0)
#pragma unroll
            for (int e = 0; e < NV; ++e) red[w * 8 + e] = a[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < NV; ++e) {
            a[e] = red[e];
            for (int v = 1; v < NTB / 64; ++v) a[e] += red[v * 8 + e];
        }
    }
}

// Column sums of a row-major [R][2K] fp32 array for the block that owns channels
// k0..k0+3 (k0 % 4 == 0): on return s[e] = sum_r rows[r][k0 + e] and
// s[4 + e] = sum_r rows[r][K + k0 + e], in every thread.  Thread t loads rows
// t, t + NTB, ... in batches of COLSUM_UN rows with all loads in flight, sums them in
// fp64 in row order, and block_sum combines the threads.
template <int NTB>
__device__ inline void colsum_pair4(const float *__restrict__ rows, int R, int K, int k0, double (&s)[8], double *red)
{
    constexpr int UN = COLSUM_UN;
    const int tid = threadIdx.x;
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0;
    for (int r0 = tid; r0 < R; r0 += NTB * UN) {
        f32x4 v[UN][2];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int r = r0 + u * NTB;
            if (r < R) {
                const float *row = rows + (size_t)r * 2 * K;
                v[u][0] = *(const f32x4 *)(row + k0);
                v[u][1] = *(const f32x4 *)(row + K + k0);
            } else {
                v[u][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                v[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[e] += (double)v[u][0][e];
                s[4 + e] += (double)v[u][1][e];
            }
    }
    block_sum<NTB, 8>(s, red);
}

// Combination of per-row statistics (count n_r, mean_r, M2_r = sum over the row's values
// of (z - mean_r)^2) into the statistics of all M values, for channels k0..k0+3 -- the
// parallel form of the variance recurrence the BatchNorm CUDA page discusses in
// section 4.3 (Chan, Golub and LeVeque's pairwise combination, applied to all rows at
// once by the law of total variance):
//   mean = (1/M) sum_r n_r mean_r,   M2 = sum_r [ M2_r + n_r (mean_r - mean)^2 ].
// rows: [R][2][K] fp32 (mean_r of the K channels, then M2_r); counts: [R] fp32 (rows
// with n_r = 0 contribute nothing).  Both sums run in fp64 in a fixed order (thread t
// takes rows t, t + NTB, ..., then block_sum), so no difference of large sums is ever
// formed.  The first batch of rows stays in registers for the second sum: up to
// NTB * COLSUM_UN rows are read from memory once.  On return mean[e] and m2[e] are
// those of channel k0 + e, in every thread.
template <int NTB>
__device__ inline void chan_combine4(const float *__restrict__ rows, const float *__restrict__ counts, int R,
                                     int K, double M, int k0, double (&mean)[4], double (&m2)[4], double *red)
{
    constexpr int UN = COLSUM_UN;
    const int tid = threadIdx.x;
    float n0[UN];
    f32x4 m0[UN], q0[UN];
    auto load = [&](int r0, float (&n)[UN], f32x4 (&m)[UN], f32x4 (&q)[UN]) {
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            const int r = r0 + u * NTB;
            if (r < R) {
                const float *row = rows + (size_t)r * 2 * K;
                n[u] = counts[r];
                m[u] = *(const f32x4 *)(row + k0);
                q[u] = *(const f32x4 *)(row + K + k0);
            } else {
                n[u] = 0.f;
                m[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                q[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    double a[4] = {0.0, 0.0, 0.0, 0.0};
    auto add_mean = [&](const float (&n)[UN], const f32x4 (&m)[UN]) {
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] += (double)n[u] * (double)m[u][e];
    };
    auto add_m2 = [&](const float (&n)[UN], const f32x4 (&m)[UN], const f32x4 (&q)[UN]) {
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double d = (double)m[u][e] - mean[e];
                a[e] += (double)q[u][e] + (double)n[u] * d * d;
            }
    };
    load(tid, n0, m0, q0);
    add_mean(n0, m0);
    for (int r0 = tid + NTB * UN; r0 < R; r0 += NTB * UN) {
        float n[UN];
        f32x4 m[UN], q[UN];
        load(r0, n, m, q);
        add_mean(n, m);
    }
    block_sum<NTB, 4>(a, red);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        mean[e] = a[e] / M;
        a[e] = 0.0;
    }
    add_m2(n0, m0, q0);
    for (int r0 = tid + NTB * UN; r0 < R; r0 += NTB * UN) {
        float n[UN];
        f32x4 m[UN], q[UN];
        load(r0, n, m, q);
        add_m2(n, m, q);
    }
    block_sum<NTB, 4>(a, red);
#pragma unroll
    for (int e = 0; e < 4; ++e) m2[e] = a[e];
}

// The BN finalize of the CBR page, section 4.2 -- with N_ac = M samples per channel,
// from the combined mean and M2 (var = M2 / M, the biased batch variance, which the page
// writes as E[z^2] - mean^2): inv_std = 1/sqrt(var + eps), eq_scale = gamma*inv_std,
// eq_bias = beta - gamma*mean*inv_std, and the running update
// next = (1 - momentum)*prev + momentum*batch (BatchNorm CUDA page, section 2.4).
// rm_out/rv_out may alias rm_in/rv_in: channel k is read before it is written.
__device__ inline void bn_finalize_channel(const BnFinalizeArgs &f, int k, double mean, double m2)
{
    double var = m2 / f.M;
    if (!(var > 0.0)) var = 0.0;
    const double invstd = 1.0 / sqrt(var + (double)f.eps);
    const double gm = (double)f.gamma[k];
    f.scale[k] = (float)(gm * invstd);
    f.shift[k] = (float)((double)f.beta[k] - gm * mean * invstd);
    f.saved_mean[k] = (float)mean;
    f.saved_invstd[k] = (float)invstd;
    const double mo = (double)f.momentum;
    const float rm = f.rm_in[k], rv = f.rv_in[k];
    f.rm_out[k] = (float)((1.0 - mo) * (double)rm + mo * mean);
    f.rv_out[k] = (float)((1.0 - mo) * (double)rv + mo * var);
}

}  // namespace cbr
