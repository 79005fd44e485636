// cbr_persist.h -- pieces shared by the persistent conv + statistics kernels (the 3x3 /
// 64-channel kernel and the first-layer kernel): 64 output channels per workgroup, eight
// waves (wave w: channel half j = w / 4, SIMD w % 4), v_mfma_f32_32x32x16_bf16 with the
// filter as A and 32 output pixels as B, so each lane holds 4 consecutive channels of one
// pixel per 8-channel group; the block epilogue (z staged in LDS as bf16, running
// per-lane statistics) and the end-of-kernel combination of the lanes' statistics into
// one (count, mean, M2) row per workgroup (the conv + genstats step of the CBR page,
// section 4.1, with the statistics in the combinable form of the BatchNorm CUDA page,
// section 4.3).
#pragma once

#include "cbr_launch.h"

namespace cbr {
namespace persist {

constexpr int NT = 512;                 // threads: 8 waves, two per SIMD
constexpr int NW = NT / 64;
constexpr int NSIMD = 4;
constexpr int HK = 64;                  // output channels
constexpr int SP = 256;                 // output pixels per step (8 blocks of 32)
constexpr int PXB = HK * 2;             // bytes per staged output pixel
constexpr int STG_BYTES = SP * PXB;     // one step's z, pixel-major
constexpr int STATS_BYTES = NW * 4 * 17 * 4;   // the end-of-kernel combination area

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Chunk permutation of a staged z pixel px: its 16-byte channel chunk c sits at position
// c ^ perm(px), so consecutive pixels' chunks spread over the LDS banks.
__device__ __forceinline__ int perm(int u) { return (u >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// v_permlane16_swap exchanges the odd 16-lane rows of a with the even rows of b: after
// it, lanes of even rows hold a of both pixels l and l + 16, lanes of odd rows b of
// pixels l - 16 and l.  Lanes l and l ^ 16 hold the same channels, so a swap and an add
// halve the registers a running per-channel sum needs.
__device__ __forceinline__ void swap_rows(float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Statistics and staging of one pixel block.  The lane holds, for pixel l32 of the
// block, channels 32j + 8g + 4hi + e in acc[4g + e] (32x32x16 layout: row
// 8*(v/4) + 4*(l/32) + v%4).  After the swap, pair i (i = 4g + e, g < 2) of lane l holds
// channel 32j + 8(g + 2 ((l / 16) % 2)) + 4hi + e of pixels l and l ^ 16 (in that order
// in even 16-lane rows, the other way round in odd ones).  Running sums s1[i], s2[i] are
// of the deviations d = z - c[i] from the lane's shift c[i], which the wave's first
// block sets to the pair's first value (the shifted-data form of the one-pass variance:
// deviations from a value of the channel do not cancel when its mean is far from zero);
// cnt counts the values summed.  With MASKED, values of pixels past the step (own: !use,
// partner: !use_p) are left out.  The bf16 results go to staging row px (16-byte chunk
// c of a row at position c ^ perm(px)).
template <bool MASKED>
__device__ __forceinline__ void epilogue(const f32x16 &acc, bool use, bool use_p, bool first, uint8_t *stg, int px,
                                         int j, int hi, float (&c)[8], float (&s1)[8], float (&s2)[8], float &cnt)
{
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = acc[k];
#pragma unroll
    for (int g = 0; g < 4; ++g)
        *(u32x2 *)(stg + px * PXB + (((4 * j + g) ^ perm(px)) << 4) + 8 * hi) =
            u32x2{pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3])};
    const bool even = (px & 16) == 0;
    const bool ua = even ? use : use_p, ub = even ? use_p : use;
#pragma unroll
    for (int i = 0; i < 8; ++i) swap_rows(v[i], v[i + 8]);
    if (first) {
        // a pixel past the step holds the conv output of the step's first pixel: a value
        // of the channel all the same
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = v[i];
    }
    // both values of pair i are the same channel: their deviations go to s1, their
    // squares to s2 (two fused multiply-adds)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float a = v[i] - c[i], b = v[i + 8] - c[i];
        if constexpr (MASKED) {
            a = ua ? a : 0.f;
            b = ub ? b : 0.f;
        }
        s1[i] += a + b;
        s2[i] = fmaf(b, b, fmaf(a, a, s2[i]));
    }
    if constexpr (MASKED)
        cnt += (float)ua + (float)ub;
    else
        cnt += 2.f;
}

// A staged step awaiting its stores: d[k] holds run k of the half being stored (a run is
// 1 KB, pixels 8q .. 8q + 7); nq runs in all, bound for zr.
struct Staged {
    u32x4 d[4];
    int nq;                          // 0: nothing staged
    __amdgpu_buffer_rsrc_t zr;
};

// The end of a persistent kernel: combines every lane's running statistics (count n,
// mean = c + s1/n, M2 = s2 - s1^2/n) by the law of total variance, mean = sum n_l mean_l
// / n, M2 = sum [M2_l + n_l (mean_l - mean)^2]: first over the 16 lanes of a 16-lane
// row, which hold the same channels (butterflies of lane shuffles, fp32; the two operands
// of every addition are the same at both lanes, so the sums are identical across the
// row), then over the 4 waves of a channel half in fp64, one thread per channel.  Writes
// row `row` of the partials (means then M2 of the 64 channels; the count at
// partials[rows * 128 + row]).  lds: STATS_BYTES of LDS no wave uses any more (every
// wave must be past its last use of it: the caller's barrier).  Called by every thread.
__device__ __forceinline__ void store_stat_row(uint8_t *lds, const float (&c)[8], const float (&s1)[8],
                                               const float (&s2)[8], float cnt, float *partials, int row, int rows)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float *st = (float *)lds;             // [NW][4][17]: wave, 16-lane row, (count, 8 means, 8 M2)
    {
        const float rc = cnt > 0.f ? 1.f / cnt : 0.f;
        float ml[8], q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ml[i] = c[i] + s1[i] * rc;
            q[i] = fmaxf(s2[i] - s1[i] * s1[i] * rc, 0.f);
        }
        auto rowsum = [](float v) {
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off);
            return v;
        };
        const float nr = rowsum(cnt);
        const float rn = nr > 0.f ? 1.f / nr : 0.f;
        float mr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) mr[i] = rowsum(cnt * ml[i]) * rn;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float d = ml[i] - mr[i];
            q[i] = rowsum(fmaf(cnt * d, d, q[i]));
        }
        if ((lane & 15) == 0) {
            float *e = st + (wave * 4 + (lane >> 4)) * 17;
            e[0] = nr;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[1 + i] = mr[i];
                e[9 + i] = q[i];
            }
        }
    }
    __syncthreads();
    if (tid < HK) {
        // channel k = 32j + 8g + 4h + e lives in waves 4j .. 4j + 3, 16-lane row 2h + g/2,
        // pair i = 4 (g % 2) + e
        const int k = tid;
        const int jk = k >> 5, g = (k >> 3) & 3, h = (k >> 2) & 1, e = k & 3;
        const int r = 2 * h + (g >> 1), i = 4 * (g & 1) + e;
        double n = 0.0, sm = 0.0;
#pragma unroll
        for (int w = 0; w < NSIMD; ++w) {
            const float *en = st + ((4 * jk + w) * 4 + r) * 17;
            n += (double)en[0];
            sm += (double)en[0] * (double)en[1 + i];
        }
        const double mean = n > 0.0 ? sm / n : 0.0;
        double m2 = 0.0;
#pragma unroll
        for (int w = 0; w < NSIMD; ++w) {
            const float *en = st + ((4 * jk + w) * 4 + r) * 17;
            const double d = (double)en[1 + i] - mean;
            m2 += (double)en[9 + i] + (double)en[0] * d * d;
        }
        float *out = partials + (size_t)row * 2 * HK;
        out[k] = (float)mean;
        out[HK + k] = (float)m2;
        if (k == 0) partials[(size_t)rows * 2 * HK + row] = (float)n;
    }
}

}  // namespace persist
}  // namespace cbr
