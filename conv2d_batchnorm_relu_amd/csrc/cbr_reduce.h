// cbr_reduce.h -- per-channel column sums of a row-major [R][2K] float partials array
// (row r: K sums, then K sums of a second quantity), accumulated in fp64 in a fixed
// order, so results are reproducible bit for bit; and the BN finalize of one channel.
#pragma once

#include "cbr_launch.h"

namespace cbr {

// Threads per block of the column-sum kernels: one wave for up to COLSUM_SMALL_R rows
// (fewer tree levels and barriers), four waves for more rows.
constexpr int COLSUM_NT_SMALL = 64, COLSUM_NT_LARGE = 256, COLSUM_SMALL_R = 1024;

// Called by all NTB threads of a block that owns channels k0..k0+3 (k0 % 4 == 0).
// Thread t sums rows t, t + NTB, ... of columns k0..k0+3 and K+k0..K+k0+3 (eight 16-byte
// loads in flight at a time), then a fixed halving tree over the threads combines them.
// red (LDS) holds NTB * 8 doubles; on return red[e] (e < 4) is the sum of column
// k0 + e and red[4 + e] that of column K + k0 + e, visible to every thread.
template <int NTB>
__device__ inline void colsum_pair4(const float *__restrict__ rows, int R, int K, int k0, double *red)
{
    constexpr int UN = 8;
    const int tid = threadIdx.x;
    double a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = 0.0;
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
                a[e] += (double)v[u][0][e];
                a[4 + e] += (double)v[u][1][e];
            }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tid * 8 + e] = a[e];
    __syncthreads();
    for (int s = NTB / 2; s > 0; s >>= 1) {
        if (tid < s)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[tid * 8 + e] += red[(tid + s) * 8 + e];
        __syncthreads();
    }
}

// The BN finalize of the CBR page, section 4.2 -- with N_ac = M samples per channel:
// mean = sum/M, var = sumsq/M - mean^2 (clamped at 0; fp64 keeps the difference
// accurate), inv_std = 1/sqrt(var + eps), eq_scale = gamma*inv_std,
// eq_bias = beta - gamma*mean*inv_std, and the running update
// next = (1 - momentum)*prev + momentum*batch (BatchNorm CUDA page, section 2.4).
// rm_out/rv_out may alias rm_in/rv_in: channel k is read before it is written.
__device__ inline void bn_finalize_channel(const BnFinalizeArgs &f, int k, double s1, double s2)
{
    const double mean = s1 / f.M;
    double var = s2 / f.M - mean * mean;
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
