// cbr_common.h -- device-side types and helpers shared by the CBR kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Geometry of one convolution as the kernels see it.  "Input" and "filter" are in the
// sense of the convolution being run (for the data gradient the input is dz and the
// filter the flipped, transposed weights).
struct ConvGeom {
    int N, H, W, C;   // input NHWC
    int K, R, S;      // filter KRSC, K = output channels
    int sh, sw, ph, pw;
    int P, Q;         // output height, width
    int M;            // N*P*Q output pixels (GEMM rows)
    int Kg;           // R*S*C (GEMM reduction length)
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bfloat16 pair (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Round-to-nearest-even float -> bfloat16 bit pattern.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b)
{
    return __uint_as_float(b << 16);
}

// Low / high bf16 of a packed 32-bit word, widened to float.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// dZ of eight consecutive channels of one pixel, the ReLU-masked BN backward of the CBR
// page (section 5.1; BatchNorm CUDA page, section 3.1): with g = dy * mask and
// xhat = (z - mean) * invstd, dz = ca * (g - cb - xhat * cg), where ca = gamma * invstd,
// cb = dbeta / M, cg = dgamma / M; rounded to bf16.  dv, zv: the chunk's bf16 dy and z;
// mk: its mask byte (bit e for channel e).  The apply kernel and the fused gradient
// prologues all call this, so dz has the same bits wherever it is formed.
__device__ __forceinline__ u32x4 bnbwd_dz8(u32x4 dv, u32x4 zv, uint32_t mk, const float (&mu)[8],
                                           const float (&is)[8], const float (&ca)[8], const float (&cb)[8],
                                           const float (&cg)[8])
{
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int e0 = 2 * h, e1 = 2 * h + 1;
        const float g0 = ((mk >> e0) & 1u) ? bf16_lo(dv[h]) : 0.f;
        const float g1 = ((mk >> e1) & 1u) ? bf16_hi(dv[h]) : 0.f;
        const float x0 = (bf16_lo(zv[h]) - mu[e0]) * is[e0];
        const float x1 = (bf16_hi(zv[h]) - mu[e1]) * is[e1];
        const float d0 = ca[e0] * (g0 - cb[e0] - x0 * cg[e0]);
        const float d1 = ca[e1] * (g1 - cb[e1] - x1 * cg[e1]);
        o[h] = pack_bf16x2(d0, d1);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

// The five per-channel coefficient vectors of bnbwd_dz8 for channels k0..k0+7, read
// from a [5][ld] table (mean, invstd, ca, cb, cg) in any address space.
template <typename T>
__device__ __forceinline__ void bnbwd_coef8(const T *tab, int ld, int k0, float (&mu)[8], float (&is)[8],
                                            float (&ca)[8], float (&cb)[8], float (&cg)[8])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        mu[e] = tab[k0 + e];
        is[e] = tab[ld + k0 + e];
        ca[e] = tab[2 * ld + k0 + e];
        cb[e] = tab[3 * ld + k0 + e];
        cg[e] = tab[4 * ld + k0 + e];
    }
}
