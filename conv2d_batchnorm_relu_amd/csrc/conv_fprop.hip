// conv_fprop.hip -- NHWC bf16 implicit-GEMM convolution on gfx950 MFMA.
//
// GEMM view: rows are output pixels m = (n,p,q), columns output channels k, reduction
// over kk = (r,s,c) with c fastest (KRSC filter rows are contiguous in kk).  A workgroup
// of four wave64s computes a BM x BN tile; each K-step stages a BM x 64 slice of the
// implicit im2col matrix and a BN x 64 slice of the filter through LDS (double
// buffered, 16-byte rows padded to 144 bytes so the fragment reads are conflict-free)
// and runs v_mfma_f32_16x16x32_bf16 with fp32 accumulators.
//
// Epilogues (one template parameter):
//   EPI_STATS      store z as bf16 and, from the fp32 accumulators, the per-channel
//                  sum and sum of squares of this tile's rows -- the conv + genstats step
//                  of the CBR page's training forward (section 4.1), which spares the
//                  statistics pass a re-read of z;
//   EPI_BIAS_RELU  y = max(acc + bias, 0) -- the folded-BN inference form (CBR page
//                  sections 2 and 6; the TileLang page's fused-ReLU epilogue);
//   EPI_PLAIN      store acc as bf16 (data gradient).
// The im2col tiling follows the TileLang page's basic convolution (grid over output
// pixel tiles x output channel tiles, a pipelined loop over ceil(KH*KW*C / block_K)).
#include "cbr_launch.h"

namespace cbr {
namespace {

constexpr int NT = 256;        // threads per workgroup: four wave64s in a 2 x 2 grid
constexpr int BK = 64;         // reduction elements per K-step
constexpr int LDK = BK + 8;    // LDS row stride (elements): 144 bytes

struct ConvParams {
    ConvGeom g;
    const uint16_t *x;
    const uint16_t *w;
    const float *bias;
    uint16_t *out;
    float *partials;
};

template <int BM, int BN, bool VEC, int EPI>
__global__ __launch_bounds__(NT) void conv_fprop_kernel(ConvParams prm)
{
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 16, NJ = WN / 16;
    constexpr int GPR = BK / 8;             // 16-byte groups per staged row
    constexpr int RPP = NT / GPR;           // rows covered per load pass
    constexpr int AI = BM / RPP, BI = BN / RPP;
    constexpr int STAGE = (BM + BN) * LDK;
    constexpr int LDO = BN + 8;             // epilogue tile row stride (elements)
    static_assert(BM * LDO <= 2 * STAGE, "epilogue tile must fit the staging buffers");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ float sstat[2][2][BN];

    const ConvGeom &g = prm.g;
    const uint16_t *__restrict__ x = prm.x;
    const uint16_t *__restrict__ wt = prm.w;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tile_m = blockIdx.x, tile_n = blockIdx.y;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int grp = tid % GPR;
    const int rbase = tid / GPR;
    const int PQ = g.P * g.Q;

    int a_hb[AI], a_wb[AI], a_nb[AI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const int m = m0 + rbase + RPP * j;
        if (m < g.M) {
            const int n = m / PQ, rem = m - n * PQ;
            const int p = rem / g.Q, q = rem - p * g.Q;
            a_hb[j] = p * g.sh - g.ph;
            a_wb[j] = q * g.sw - g.pw;
            a_nb[j] = n * g.H * g.W * g.C;
        } else {
            a_hb[j] = 0; a_wb[j] = 0; a_nb[j] = -1;
        }
    }

    u32x4 ra[AI], rb[BI];
    auto load = [&](int ks) {
        const int kk0 = ks * BK + grp * 8;
        if constexpr (VEC) {
            int r = 0, s = 0, c0 = 0;
            const bool kok = kk0 < g.Kg;
            if (kok) {
                const int tap = kk0 / g.C;
                c0 = kk0 - tap * g.C;
                r = tap / g.S;
                s = tap - r * g.S;
            }
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                const int h = a_hb[j] + r, w = a_wb[j] + s;
                const bool ok = kok && a_nb[j] >= 0 && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
                ra[j] = ok ? *(const u32x4 *)(x + a_nb[j] + (h * g.W + w) * g.C + c0) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < BI; ++j) {
                const int k = n0 + rbase + RPP * j;
                const bool ok = kok && k < g.K;
                rb[j] = ok ? *(const u32x4 *)(wt + (size_t)k * g.Kg + kk0) : u32x4{0, 0, 0, 0};
            }
        } else {
            int er[8], es[8], ec[8];
            bool eok[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = kk0 + e;
                eok[e] = kk < g.Kg;
                const int tap = eok[e] ? kk / g.C : 0;
                ec[e] = eok[e] ? kk - tap * g.C : 0;
                er[e] = tap / g.S;
                es[e] = tap - er[e] * g.S;
            }
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                uint32_t v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int h = a_hb[j] + er[e], w = a_wb[j] + es[e];
                    const bool ok = eok[e] && a_nb[j] >= 0 && (unsigned)h < (unsigned)g.H &&
                                    (unsigned)w < (unsigned)g.W;
                    v[e] = ok ? x[a_nb[j] + (h * g.W + w) * g.C + ec[e]] : 0u;
                }
                ra[j] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
            }
#pragma unroll
            for (int j = 0; j < BI; ++j) {
                const int k = n0 + rbase + RPP * j;
                uint32_t v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (eok[e] && k < g.K) ? wt[(size_t)k * g.Kg + kk0 + e] : 0u;
                rb[j] = u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
            }
        }
    };
    auto store = [&](int buf) {
        uint16_t *sa = smem + buf * STAGE;
        uint16_t *sb = sa + BM * LDK;
#pragma unroll
        for (int j = 0; j < AI; ++j) *(u32x4 *)(sa + (rbase + RPP * j) * LDK + grp * 8) = ra[j];
#pragma unroll
        for (int j = 0; j < BI; ++j) *(u32x4 *)(sb + (rbase + RPP * j) * LDK + grp * 8) = rb[j];
    };

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const uint16_t *sa = smem + buf * STAGE;
        const uint16_t *sb = sa + BM * LDK;
#pragma unroll
        for (int kh = 0; kh < BK / 32; ++kh) {
            bf16x8 a[MI], b[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                a[i] = *(const bf16x8 *)(sa + (wm * WM + 16 * i + (lane & 15)) * LDK + kh * 32 + (lane >> 4) * 8);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                b[j] = *(const bf16x8 *)(sb + (wn * WN + 16 * j + (lane & 15)) * LDK + kh * 32 + (lane >> 4) * 8);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    const int ksteps = (g.Kg + BK - 1) / BK;
    load(0);
    store(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < ksteps) load(ks + 1);
        compute(cur);
        if (ks + 1 < ksteps) store(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator layout of v_mfma_f32_16x16x32: lane l holds column
    // (l & 15) and rows 4*(l >> 4) + v, v = 0..3, of each 16 x 16 block.
    if constexpr (EPI == EPI_STATS) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float a = acc[i][j][v];
                    s1 += a;
                    s2 += a * a;
                }
            s1 += __shfl_xor(s1, 16);
            s2 += __shfl_xor(s2, 16);
            s1 += __shfl_xor(s1, 32);
            s2 += __shfl_xor(s2, 32);
            if (lane < 16) {
                sstat[wm][0][wn * WN + 16 * j + lane] = s1;
                sstat[wm][1][wn * WN + 16 * j + lane] = s2;
            }
        }
    }
    float bcol[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int col = n0 + wn * WN + 16 * j + (lane & 15);
        bcol[j] = (EPI == EPI_BIAS_RELU && col < g.K) ? prm.bias[col] : 0.f;
    }
    uint16_t *so = smem;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = wm * WM + 16 * i + 4 * (lane >> 4) + v;
                const int col = wn * WN + 16 * j + (lane & 15);
                float val = acc[i][j][v];
                if constexpr (EPI == EPI_BIAS_RELU) val = fmaxf(val + bcol[j], 0.f);
                so[row * LDO + col] = (uint16_t)f32_to_bf16_bits(val);
            }
    __syncthreads();
    if constexpr (EPI == EPI_STATS) {
        if (tid < BN && n0 + tid < g.K) {
            float *pt = prm.partials + (size_t)tile_m * 2 * g.K;
            pt[n0 + tid] = sstat[0][0][tid] + sstat[1][0][tid];
            pt[g.K + n0 + tid] = sstat[0][1][tid] + sstat[1][1][tid];
        }
    }
    constexpr int CPRO = BN / 8;
    for (int idx = tid; idx < BM * CPRO; idx += NT) {
        const int row = idx / CPRO, ch = idx - row * CPRO;
        const int m = m0 + row, k = n0 + ch * 8;
        if (m >= g.M || k >= g.K) continue;
        if ((g.K & 7) == 0) {
            *(u32x4 *)(prm.out + (size_t)m * g.K + k) = *(const u32x4 *)(so + row * LDO + ch * 8);
        } else {   // output rows not 16-byte aligned (data gradient with C % 8 != 0)
            for (int e = 0; e < 8 && k + e < g.K; ++e) prm.out[(size_t)m * g.K + k + e] = so[row * LDO + ch * 8 + e];
        }
    }
}

template <int BM, int BN, bool VEC>
hipError_t launch_epi(int epi, const ConvParams &prm, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    switch (epi) {
    case EPI_STATS: return launch(conv_fprop_kernel<BM, BN, VEC, EPI_STATS>, grid, dim3(NT), 0, st, e0, e1, prm);
    case EPI_BIAS_RELU:
        return launch(conv_fprop_kernel<BM, BN, VEC, EPI_BIAS_RELU>, grid, dim3(NT), 0, st, e0, e1, prm);
    default: return launch(conv_fprop_kernel<BM, BN, VEC, EPI_PLAIN>, grid, dim3(NT), 0, st, e0, e1, prm);
    }
}

}  // namespace

ConvPlan conv_plan(const ConvGeom &g)
{
    ConvPlan p;
    p.bm = 128;
    p.bn = (g.K >= 128) ? 128 : 64;
    p.vec = (g.C % 8) == 0;
    p.tiles_m = (g.M + p.bm - 1) / p.bm;
    p.tiles_n = (g.K + p.bn - 1) / p.bn;
    return p;
}

hipError_t launch_conv_fprop(const ConvGeom &g, int epi, const uint16_t *x, const uint16_t *w,
                             const float *bias, uint16_t *out, float *partials, hipStream_t st, hipEvent_t e0,
                             hipEvent_t e1)
{
    const ConvPlan p = conv_plan(g);
    ConvParams prm{g, x, w, bias, out, partials};
    dim3 grid(p.tiles_m, p.tiles_n);
    if (p.bn == 128) {
        return p.vec ? launch_epi<128, 128, true>(epi, prm, grid, st, e0, e1)
                     : launch_epi<128, 128, false>(epi, prm, grid, st, e0, e1);
    }
    return p.vec ? launch_epi<128, 64, true>(epi, prm, grid, st, e0, e1)
                 : launch_epi<128, 64, false>(epi, prm, grid, st, e0, e1);
}

}  // namespace cbr
