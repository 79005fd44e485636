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
