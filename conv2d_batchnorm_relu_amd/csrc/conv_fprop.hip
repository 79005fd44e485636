// conv_fprop.hip -- NHWC bf16 implicit-GEMM convolution on gfx950 MFMA.
//
// GEMM view: rows are output pixels m = (n,p,q), columns output channels k, reduction
// over kk = (r,s,c) with c fastest (KRSC filter rows are contiguous in kk).  A workgroup
// of four wave64s computes a BM x BN tile; each K-step stages a BM x 64 slice of the
// implicit im2col matrix and a BN x 64 slice of the filter through LDS (double
// buffered, rows padded to 144 bytes so the fragment reads are conflict-free) and runs
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  The global loads of a K-step are
// issued two K-steps ahead (two register stages), so their latency is covered by two
// K-steps of MFMAs of this workgroup and of the other workgroup sharing the CU.
//
// Epilogues (one template parameter):
//   EPI_STATS      store z as bf16 and, from the fp32 accumulators, the per-channel
//                  statistics of this tile's rows (count, mean, and M2 = the sum of
//                  squared deviations from that mean, by two passes over the registers)
//                  -- the conv + genstats step of the CBR page's training forward
//                  (section 4.1), which spares the statistics pass a re-read of z;
//   EPI_BIAS_RELU  y = max(acc + bias, 0) -- the folded-BN inference form (CBR page
//                  sections 2 and 6; the TileLang page's fused-ReLU epilogue);
//   EPI_PLAIN      store acc as bf16 (data gradient);
//   EPI_BIAS       y = acc + bias (Conv2D with bias, no activation).
// A NULL bias reads as zeros.
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
    // FUSE: the input is dz, formed on load from the backward's dy, z, mask and its
    // [5][C] coefficient table (x unused)
    const uint16_t *dy, *z;
    const uint8_t *mask;
    const float *bnc;
};

// Channels of dz the fused form's coefficient table holds in LDS.
constexpr int FUSE_MAXC = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Gather modes of the implicit im2col rows.
//   GATHER_SCALAR  C % 8 != 0: element loads (first layers that no special kernel takes);
//   GATHER_VEC     C % 8 == 0: 16-byte loads, each thread decodes its own tap;
//   GATHER_TAP     C % 64 == 0: a K-step lies inside one filter tap, so the tap and its
//                  offset are uniform and each thread adds them to a per-row base.
// The vector modes load through bounds-checked buffer resources: a padding position
// or a row past M gets an offset past the end and reads zeros, with no branch.
enum { GATHER_SCALAR = 0, GATHER_VEC = 1, GATHER_TAP = 2 };
constexpr uint32_t OOB = 0x80000000u;   // past the end of every buffer (sizes < 2^31)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// FUSE (the data gradient of a backward that keeps no dz tensor): the A operand is dz,
// formed while staging from dy, the stored z and the ReLU mask (bnbwd_dz8, the same
// arithmetic as the BN-backward apply), zero at padding positions.
template <int BM, int BN, int MODE, int EPI, bool FUSE = false>
__global__ __launch_bounds__(NT, 2) void conv_fprop_kernel(ConvParams prm)
{
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 32, NJ = WN / 32;
    constexpr int GPR = BK / 8;             // 16-byte groups per staged row
    constexpr int RPP = NT / GPR;           // rows covered per load pass
    constexpr int AI = BM / RPP, BI = BN / RPP;
    constexpr int STAGE = (BM + BN) * LDK;
    constexpr int LDO = BN + 8;             // epilogue tile row stride (elements)
    static_assert(BM * LDO <= 2 * STAGE, "epilogue tile must fit the staging buffers");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ float sstat[2][2][BN];
    __shared__ __attribute__((aligned(16))) float sbn[FUSE ? 5 * FUSE_MAXC : 4];
    static_assert(!FUSE || MODE != GATHER_SCALAR, "the fused form gathers 16-byte channel chunks");

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

    constexpr bool VEC = MODE != GATHER_SCALAR;
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
            a_hb[j] = -0x40000000; a_wb[j] = 0; a_nb[j] = -1;   // never inside the image
        }
    }
    const uint32_t xbytes = (uint32_t)((size_t)g.N * g.H * g.W * g.C * 2);
    const __amdgpu_buffer_rsrc_t xr = rsrc_of(FUSE ? prm.dy : x, xbytes);
    const __amdgpu_buffer_rsrc_t zr = rsrc_of(prm.z, FUSE ? xbytes : 0u);
    const __amdgpu_buffer_rsrc_t mr = rsrc_of(prm.mask, FUSE ? xbytes / 16 : 0u);
    if constexpr (FUSE) {
        for (int i = tid; i < 5 * g.C; i += NT) sbn[i] = prm.bnc[i];
        __syncthreads();
    }
    const __amdgpu_buffer_rsrc_t wr = rsrc_of(wt, (uint32_t)((size_t)g.K * g.Kg * 2));
    // Byte offset of each A row's pixel (tap 0, channel grp*8) and each B row's start.
    int a_off[AI], b_off[AI > BI ? AI : BI];
#pragma unroll
    for (int j = 0; j < AI; ++j) a_off[j] = a_nb[j] >= 0 ? 2 * (a_nb[j] + (a_hb[j] * g.W + a_wb[j]) * g.C + grp * 8) : 0;
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int k = n0 + rbase + RPP * j;
        b_off[j] = k < g.K ? 2 * (k * g.Kg + grp * 8) : (int)OOB;
    }

    u32x4 ra2[2][AI], rb2[2][BI];
    // FUSE: the z chunks and mask bytes beside the dy chunks in ra2, and which rows are
    // inside the image (bit j)
    u32x4 rz2[2][FUSE ? AI : 1];
    uint32_t rm2[2][FUSE ? AI : 1], okm2[2] = {0u, 0u};
    auto load_a = [&](int set, int j, bool ok, int off, u32x4 (&ra)[AI]) {
        ra[j] = __builtin_amdgcn_raw_buffer_load_b128(xr, ok ? off : (int)OOB, 0, 0);
        if constexpr (FUSE) {
            rz2[set][j] = __builtin_amdgcn_raw_buffer_load_b128(zr, ok ? off : (int)OOB, 0, 0);
            rm2[set][j] = __builtin_amdgcn_raw_buffer_load_b8(mr, ok ? off >> 4 : (int)OOB, 0, 0);
            okm2[set] = ok ? okm2[set] | (1u << j) : okm2[set] & ~(1u << j);
        }
    };
    auto load = [&](int ks, u32x4 (&ra)[AI], u32x4 (&rb)[BI]) {
        const int set = &ra == &ra2[0] ? 0 : 1;
        const int kk0 = ks * BK + grp * 8;
        if constexpr (MODE == GATHER_TAP) {
            // Uniform tap (r, s) and channel base of this K-step.
            const int kb = ks * BK;
            const int tap = kb / g.C, c0b = kb - tap * g.C;
            const int r = tap / g.S, s = tap - r * g.S;
            const int toff = 2 * ((r * g.W + s) * g.C + c0b);
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                const int h = a_hb[j] + r, w = a_wb[j] + s;
                const bool ok = (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
                load_a(set, j, ok, a_off[j] + toff, ra);
            }
#pragma unroll
            for (int j = 0; j < BI; ++j)
                rb[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, b_off[j] < 0 ? (int)OOB : b_off[j] + 2 * kb, 0, 0);
        } else if constexpr (VEC) {
            int r = 0, s = 0, c0 = 0;
            const bool kok = kk0 < g.Kg;
            if (kok) {
                const int tap = kk0 / g.C;
                c0 = kk0 - tap * g.C;
                r = tap / g.S;
                s = tap - r * g.S;
            }
            const int toff = 2 * ((r * g.W + s) * g.C + c0 - grp * 8);
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                const int h = a_hb[j] + r, w = a_wb[j] + s;
                const bool ok = kok && (unsigned)h < (unsigned)g.H && (unsigned)w < (unsigned)g.W;
                load_a(set, j, ok, a_off[j] + toff, ra);
            }
#pragma unroll
            for (int j = 0; j < BI; ++j)
                rb[j] = __builtin_amdgcn_raw_buffer_load_b128(
                    wr, (kok && b_off[j] >= 0) ? b_off[j] + 2 * ks * BK : (int)OOB, 0, 0);
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
    // ks: the k-step whose data the register set holds (FUSE: picks the dz channels)
    auto store = [&](int buf, const u32x4 (&ra)[AI], const u32x4 (&rb)[BI], int ks) {
        uint16_t *sa = smem + buf * STAGE;
        uint16_t *sb = sa + BM * LDK;
        if constexpr (FUSE) {
            const int set = &ra == &ra2[0] ? 0 : 1;
            const int kk0 = ks * BK + grp * 8;
            const int ch = kk0 < g.Kg ? kk0 - (kk0 / g.C) * g.C : 0;
            float mu[8], is[8], ca[8], cb[8], cg[8];
            bnbwd_coef8(sbn, g.C, ch, mu, is, ca, cb, cg);
#pragma unroll
            for (int j = 0; j < AI; ++j) {
                const u32x4 d = bnbwd_dz8(ra[j], rz2[set][j], rm2[set][j], mu, is, ca, cb, cg);
                *(u32x4 *)(sa + (rbase + RPP * j) * LDK + grp * 8) =
                    ((okm2[set] >> j) & 1u) ? d : u32x4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int j = 0; j < AI; ++j) *(u32x4 *)(sa + (rbase + RPP * j) * LDK + grp * 8) = ra[j];
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) *(u32x4 *)(sb + (rbase + RPP * j) * LDK + grp * 8) = rb[j];
    };

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // 32x32x16 fragments: lane l reads row (l & 31), reduction elements 8*(l >> 5)..+7
    // of the 16-element slice kh.
    // Fragments of slice kh + 1 are read while the MFMAs of slice kh run.
    auto compute = [&](int buf) {
        const uint16_t *sa = smem + buf * STAGE;
        const uint16_t *sb = sa + BM * LDK;
        bf16x8 a[2][MI], b[2][NJ];
        auto rd = [&](int kh, int d) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
                a[d][i] = *(const bf16x8 *)(sa + (wm * WM + 32 * i + (lane & 31)) * LDK + kh * 16 + (lane >> 5) * 8);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                b[d][j] = *(const bf16x8 *)(sb + (wn * WN + 32 * j + (lane & 31)) * LDK + kh * 16 + (lane >> 5) * 8);
        };
        rd(0, 0);
#pragma unroll
        for (int kh = 0; kh < BK / 16; ++kh) {
            if (kh + 1 < BK / 16) rd(kh + 1, (kh + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kh & 1][i], b[kh & 1][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Stage ks lives in LDS buffer ks & 1 while it is computed; stage ks + 1 is in the
    // register set (ks + 1) & 1, loaded during K-step ks - 1; stage ks + 2 is loaded
    // into register set ks & 1 (free since stage ks went to LDS).
    const int ksteps = (g.Kg + BK - 1) / BK;
    load(0, ra2[0], rb2[0]);
    if (ksteps > 1) load(1, ra2[1], rb2[1]);
    store(0, ra2[0], rb2[0], 0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ks += 2) {
        if (ks + 2 < ksteps) load(ks + 2, ra2[0], rb2[0]);
        compute(0);
        if (ks + 1 < ksteps) store(1, ra2[1], rb2[1], ks + 1);
        __syncthreads();
        if (ks + 1 >= ksteps) break;
        if (ks + 3 < ksteps) load(ks + 3, ra2[1], rb2[1]);
        compute(1);
        if (ks + 2 < ksteps) store(0, ra2[0], rb2[0], ks + 2);
        __syncthreads();
    }

    // Epilogue.  Accumulator layout of v_mfma_f32_32x32x16: lane l holds column
    // (l & 31) and rows 8*(v/4) + 4*(l >> 5) + v%4, v = 0..15, of each 32 x 32 block.
    // Statistics, first pass: the column sums of the tile (rows past M hold zeros).
    const int nrows = min(BM, g.M - m0);
    if constexpr (EPI == EPI_STATS) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            float s1 = 0.f;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) s1 += acc[i][j][v];
            s1 += __shfl_xor(s1, 32);
            if (lane < 32) sstat[wm][0][wn * WN + 32 * j + lane] = s1;
        }
    }
    float bcol[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int col = n0 + wn * WN + 32 * j + (lane & 31);
        bcol[j] = ((EPI == EPI_BIAS_RELU || EPI == EPI_BIAS) && prm.bias && col < g.K) ? prm.bias[col] : 0.f;
    }
    uint16_t *so = smem;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * WM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int col = wn * WN + 32 * j + (lane & 31);
                float val = acc[i][j][v];
                if constexpr (EPI == EPI_BIAS_RELU) val = fmaxf(val + bcol[j], 0.f);
                if constexpr (EPI == EPI_BIAS) val += bcol[j];
                so[row * LDO + col] = (uint16_t)f32_to_bf16_bits(val);
            }
    __syncthreads();
    // Second pass: the squared deviations of the valid rows from the tile's column means.
    auto tile_mean = [&](int col) { return (sstat[0][0][col] + sstat[1][0][col]) / (float)nrows; };
    if constexpr (EPI == EPI_STATS) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float mt = tile_mean(wn * WN + 32 * j + (lane & 31));
            float s2 = 0.f;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * WM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    const float d = acc[i][j][v] - mt;
                    s2 = row < nrows ? fmaf(d, d, s2) : s2;
                }
            s2 += __shfl_xor(s2, 32);
            if (lane < 32) sstat[wm][1][wn * WN + 32 * j + lane] = s2;
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
    if constexpr (EPI == EPI_STATS) {
        // Row tile_m of the partials: means, M2, and (after all rows) the row's count.
        __syncthreads();
        if (tid < BN && n0 + tid < g.K) {
            float *pt = prm.partials + (size_t)tile_m * 2 * g.K;
            pt[n0 + tid] = tile_mean(tid);
            pt[g.K + n0 + tid] = sstat[0][1][tid] + sstat[1][1][tid];
        }
        if (tile_n == 0 && tid == 0) prm.partials[(size_t)gridDim.x * 2 * g.K + tile_m] = (float)nrows;
    }
}

template <int BM, int BN, int MODE>
hipError_t launch_epi(int epi, const ConvParams &prm, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    switch (epi) {
    case EPI_STATS: return launch(conv_fprop_kernel<BM, BN, MODE, EPI_STATS>, grid, dim3(NT), 0, st, e0, e1, prm);
    case EPI_BIAS_RELU:
        return launch(conv_fprop_kernel<BM, BN, MODE, EPI_BIAS_RELU>, grid, dim3(NT), 0, st, e0, e1, prm);
    case EPI_BIAS: return launch(conv_fprop_kernel<BM, BN, MODE, EPI_BIAS>, grid, dim3(NT), 0, st, e0, e1, prm);
    default: return launch(conv_fprop_kernel<BM, BN, MODE, EPI_PLAIN>, grid, dim3(NT), 0, st, e0, e1, prm);
    }
}

template <int BM, int BN>
hipError_t launch_mode(const ConvGeom &g, int epi, const ConvParams &prm, dim3 grid, hipStream_t st, hipEvent_t e0,
                       hipEvent_t e1)
{
    if (g.C % 64 == 0) return launch_epi<BM, BN, GATHER_TAP>(epi, prm, grid, st, e0, e1);
    if (g.C % 8 == 0) return launch_epi<BM, BN, GATHER_VEC>(epi, prm, grid, st, e0, e1);
    return launch_epi<BM, BN, GATHER_SCALAR>(epi, prm, grid, st, e0, e1);
}

}  // namespace

hipError_t launch_conv_dgrad_fused(const ConvGeom &d, const uint16_t *dy, const uint16_t *z, const uint8_t *mask,
                                   const float *bnc, const uint16_t *wt, uint16_t *dx, hipStream_t st, hipEvent_t e0,
                                   hipEvent_t e1)
{
    // 128 x 64 tiles: the 128 x 128 form holds too many registers with the dz staging
    const ConvPlan p = conv_plan(d, PLAN_GEN_128X64);
    ConvParams prm{d, nullptr, wt, nullptr, dx, nullptr, dy, z, mask, bnc};
    dim3 grid(p.tiles_m, p.tiles_n);
    return d.C % 64 == 0
               ? launch(conv_fprop_kernel<128, 64, GATHER_TAP, EPI_PLAIN, true>, grid, dim3(NT), 0, st, e0, e1, prm)
               : launch(conv_fprop_kernel<128, 64, GATHER_VEC, EPI_PLAIN, true>, grid, dim3(NT), 0, st, e0, e1, prm);
}

ConvPlan conv_plan(const ConvGeom &g, int plan)
{
    ConvPlan p;
    p.bm = 128;
    p.bn = plan == PLAN_GEN_128X64 ? 64 : 128;
    p.vec = (g.C % 8) == 0;
    p.tiles_m = (g.M + p.bm - 1) / p.bm;
    p.tiles_n = (g.K + p.bn - 1) / p.bn;
    return p;
}

hipError_t launch_conv_fprop(const ConvGeom &g, int epi, int plan, const uint16_t *x, const uint16_t *w,
                             const float *bias, uint16_t *out, float *partials, hipStream_t st, hipEvent_t e0,
                             hipEvent_t e1)
{
    if (plan == PLAN_IG_224X256 || plan == PLAN_IG_448X128)
        return launch_conv_igemm(g, epi, plan, x, w, bias, out, partials, st, e0, e1);
    const ConvPlan p = conv_plan(g, plan);
    ConvParams prm{g, x, w, bias, out, partials, nullptr, nullptr, nullptr, nullptr};
    dim3 grid(p.tiles_m, p.tiles_n);
    if (p.bn == 128) return launch_mode<128, 128>(g, epi, prm, grid, st, e0, e1);
    return launch_mode<128, 64>(g, epi, prm, grid, st, e0, e1);
}

}  // namespace cbr
