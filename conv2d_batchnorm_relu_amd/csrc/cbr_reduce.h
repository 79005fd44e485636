// cbr_reduce.h -- block-wide column sums of a row-major [R][K2] array (float or double
// rows), accumulated in fp64 in a fixed order, so results are reproducible bit for bit.
#pragma once

#include "cbr_common.h"

namespace cbr {

// All 256 threads of the block call this.  When the 16-byte column count of a row
// divides 256, each thread owns one 16-byte column and a fixed set of rows, and issues
// 16 independent loads before adding any of them (one memory latency per 16 rows of
// its set, not one per row).  tot (LDS, K2 doubles) receives the sums; scratch (LDS)
// needs 256 * 16 / sizeof(TIn) doubles.  Ends with a barrier.
template <typename TIn>
__device__ void sum_rows_to_lds(const TIn *__restrict__ in, int R, int K2, double *tot, double *scratch)
{
    constexpr int NTH = 256;
    constexpr int VPL = 16 / (int)sizeof(TIn);
    constexpr int UN = 16;
    const int tid = threadIdx.x;
    const int cols = K2 / VPL;
    if (K2 % VPL == 0 && cols <= NTH && NTH % cols == 0) {
        const int col = tid % cols, rg = tid / cols, ngr = NTH / cols;
        double acc[VPL];
#pragma unroll
        for (int e = 0; e < VPL; ++e) acc[e] = 0.0;
        for (int r0 = rg; r0 < R; r0 += ngr * UN) {
            TIn v[UN][VPL];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                const int r = r0 + u * ngr;
                if (r < R) {
                    const TIn *src = in + (size_t)r * K2 + col * VPL;
#pragma unroll
                    for (int e = 0; e < VPL; ++e) v[u][e] = src[e];
                } else {
#pragma unroll
                    for (int e = 0; e < VPL; ++e) v[u][e] = (TIn)0;
                }
            }
#pragma unroll
            for (int u = 0; u < UN; ++u)
#pragma unroll
                for (int e = 0; e < VPL; ++e) acc[e] += (double)v[u][e];
        }
#pragma unroll
        for (int e = 0; e < VPL; ++e) scratch[rg * K2 + col * VPL + e] = acc[e];
        __syncthreads();
        for (int k2 = tid; k2 < K2; k2 += NTH) {
            double s = 0.0;
            for (int g = 0; g < ngr; ++g) s += scratch[g * K2 + k2];
            tot[k2] = s;
        }
    } else {
        for (int k2 = tid; k2 < K2; k2 += NTH) {
            double s = 0.0;
            for (int r = 0; r < R; ++r) s += (double)in[(size_t)r * K2 + k2];
            tot[k2] = s;
        }
    }
    __syncthreads();
}

}  // namespace cbr
