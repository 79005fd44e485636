// conv_wgrad.hip -- convolution weight gradient and the filter flip of the data gradient.
//
// Weight gradient (CBR page, section 5.2, WGrad from dL/d(conv_out) and X; the Burn
// page's backward, grad_rhs = lhs^T * grad, is its GEMM form):
//   dw[k][kk] = sum_m dz[m][k] * im2col(x)[m][kk],   kk = (r,s,c), m = (n,p,q).
// GEMM rows are output channels k, columns filter positions kk, and the reduction runs
// over output pixels m, which are the slow (non-contiguous) dimension of both operands.
// Each K-step loads a 64-pixel slice of dz and of im2col(x) with 16-byte channel-chunk
// loads, and writes it to LDS transposed (pixel-contiguous rows) as 32-bit pixel pairs;
// the 16-byte blocks of each LDS row are XOR-swizzled by (row/8) so that both these
// writes and the 128-bit MFMA fragment reads hit distinct banks.  The pixel range is
// split over blockIdx.z; split partials are summed in a fixed order by a second kernel
// (no atomics: results are bitwise reproducible).
#include "cbr_launch.h"

namespace cbr {
namespace {

constexpr int NT = 256;
constexpr int BKM = 64;        // output pixels per K-step
constexpr int LDK = BKM + 8;   // LDS row stride (elements)
constexpr int WGRAD_STAGES_128 = 1;   // register stages of the 128 x 128 tile

// Unsigned division by a fixed divisor d >= 1 for dividends below 2^31 (round-up
// multiplier method): n / d == (umulhi(n, mul) + n) >> shift.
struct FastDiv {
    uint32_t mul, shift;
};

FastDiv fast_div(uint32_t d)
{
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return FastDiv{(uint32_t)m, s};
}

__device__ __forceinline__ uint32_t div_by(uint32_t n, FastDiv f)
{
    return (__umulhi(n, f.mul) + n) >> f.shift;
}

struct WgradParams {
    ConvGeom g;
    const uint16_t *dz;
    const uint16_t *x;
    float *out;            // [splits][K][Kg] (or dw itself when splits == 1)
    int rows_per_split;
    FastDiv dpq, dq;       // division by P*Q and by Q
    // FUSE: dz formed on load from the backward's dy, z, mask and its [5][K] coefficient
    // table (dz unused)
    const uint16_t *dy, *z;
    const uint8_t *mask;
    const float *bnc;
};

__device__ __forceinline__ int swz(int row, int m)   // element offset of (row, m) in a tile row
{
    return row * LDK + ((((m >> 3) ^ (row >> 3)) & 7) << 3) + (m & 7);
}

constexpr uint32_t OOB = 0x80000000u;   // past the end of every buffer (sizes < 2^31)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// FUSE (the weight gradient of a backward that keeps no dz tensor): the dz operand is
// formed while staging from dy, the stored z and the ReLU mask (bnbwd_dz8, the same
// arithmetic as the BN-backward apply).
template <int BMK, int BNC, bool VEC, int STAGES, bool FUSE = false>
__global__ __launch_bounds__(NT, 2) void conv_wgrad_kernel(WgradParams prm)
{
    constexpr int WM = BMK / 2, WN = BNC / 2;
    constexpr int MI = WM / 32, NJ = WN / 32;
    constexpr int AI = (BKM / 2) * (BMK / 8) / NT;   // (pixel pair, chunk) items per thread
    constexpr int BI = (BKM / 2) * (BNC / 8) / NT;
    constexpr int STAGE = (BMK + BNC) * LDK;
    static_assert(AI >= 1 && BI >= 1, "tile too small for the thread count");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const ConvGeom &g = prm.g;
    const uint16_t *__restrict__ x = prm.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int k0 = blockIdx.y * BMK, n0 = blockIdx.x * BNC;
    const int mbeg = blockIdx.z * prm.rows_per_split;
    const int mend = min(g.M, mbeg + prm.rows_per_split);
    const uint32_t zbytes = (uint32_t)((size_t)g.M * g.K * 2);
    const __amdgpu_buffer_rsrc_t dzr = rsrc_of(FUSE ? prm.dy : prm.dz, zbytes);
    const __amdgpu_buffer_rsrc_t zr = rsrc_of(prm.z, FUSE ? zbytes : 0u);
    const __amdgpu_buffer_rsrc_t mr = rsrc_of(prm.mask, FUSE ? zbytes / 16 : 0u);
    // FUSE: the coefficient table of this workgroup's BMK channels, [5][BMK]
    __shared__ __attribute__((aligned(16))) float sbn[FUSE ? 5 * BMK : 4];
    if constexpr (FUSE) {
        for (int i = tid; i < 5 * BMK; i += NT) {
            const int t = i / BMK, k = k0 + i - t * BMK;
            sbn[i] = k < g.K ? prm.bnc[t * g.K + k] : 0.f;
        }
        __syncthreads();
    }
    // FUSE: z chunks and mask bytes beside the dy chunks, and which (item, pixel) are in
    // range (bit 2j + h), per register set
    u32x4 rz2[2][FUSE ? AI : 1][2];
    uint32_t rm2[2][FUSE ? AI : 1][2], okm2[2] = {0u, 0u};
    const __amdgpu_buffer_rsrc_t xr = rsrc_of(x, (uint32_t)((size_t)g.N * g.H * g.W * g.C * 2));

    // item i -> (pixel pair p, chunk cc): within a wave, 8 pairs x 8 chunks.
    auto item_p = [](int i) { return (i & 7) + 8 * ((i >> 6) & 3); };
    auto item_c = [](int i) { return ((i >> 3) & 7) + 8 * (i >> 8); };

    // Per-thread filter-position decode of its B chunks (fixed for the whole kernel).
    int b_r[BI], b_s[BI], b_c[BI];
    bool b_ok[BI];
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int kk0 = n0 + 8 * item_c(tid + NT * j);
        b_ok[j] = kk0 < g.Kg;
        const int tap = b_ok[j] ? kk0 / g.C : 0;
        b_c[j] = b_ok[j] ? kk0 - tap * g.C : 0;
        b_r[j] = tap / g.S;
        b_s[j] = tap - b_r[j] * g.S;
    }

    auto load = [&](int mstep, int set, u32x4 (&ra)[AI][2], u32x4 (&rb)[BI][2]) {
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int it = tid + NT * j;
            const int k = k0 + 8 * item_c(it);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int m = mstep + 2 * item_p(it) + h;
                const bool ok = m < mend && k < g.K;
                const int off = ok ? 2 * (m * g.K + k) : (int)OOB;
                ra[j][h] = __builtin_amdgcn_raw_buffer_load_b128(dzr, off, 0, 0);
                if constexpr (FUSE) {
                    rz2[set][j][h] = __builtin_amdgcn_raw_buffer_load_b128(zr, off, 0, 0);
                    rm2[set][j][h] = __builtin_amdgcn_raw_buffer_load_b8(mr, ok ? off >> 4 : (int)OOB, 0, 0);
                    const uint32_t bit = 1u << (2 * j + h);
                    okm2[set] = ok ? okm2[set] | bit : okm2[set] & ~bit;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const int it = tid + NT * j;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int m = mstep + 2 * item_p(it) + h;
                const int n = (int)div_by((uint32_t)m, prm.dpq), rem = m - n * g.P * g.Q;
                const int p = (int)div_by((uint32_t)rem, prm.dq), q = rem - p * g.Q;
                const int hb = p * g.sh - g.ph, wb = q * g.sw - g.pw;
                const int nb = n * g.H * g.W * g.C;
                if constexpr (VEC) {
                    const int hh = hb + b_r[j], ww = wb + b_s[j];
                    const bool ok = m < mend && b_ok[j] && (unsigned)hh < (unsigned)g.H && (unsigned)ww < (unsigned)g.W;
                    rb[j][h] = __builtin_amdgcn_raw_buffer_load_b128(
                        xr, ok ? 2 * (nb + (hh * g.W + ww) * g.C + b_c[j]) : (int)OOB, 0, 0);
                } else {
                    const int kk0 = n0 + 8 * item_c(it);
                    uint32_t e16[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int kk = kk0 + e;
                        e16[e] = 0u;
                        if (m < mend && kk < g.Kg) {
                            const int tap = kk / g.C, c = kk - tap * g.C;
                            const int r = tap / g.S, s = tap - r * g.S;
                            const int hh = hb + r, ww = wb + s;
                            if ((unsigned)hh < (unsigned)g.H && (unsigned)ww < (unsigned)g.W)
                                e16[e] = x[nb + (hh * g.W + ww) * g.C + c];
                        }
                    }
                    rb[j][h] = u32x4{e16[0] | (e16[1] << 16), e16[2] | (e16[3] << 16), e16[4] | (e16[5] << 16),
                                     e16[6] | (e16[7] << 16)};
                }
            }
        }
    };
    // Transposed store: channel-chunk element e of pixels (2p, 2p+1) -> row 8*cc + e,
    // columns 2p and 2p+1 (one 32-bit LDS write).
    auto store = [&](int buf, int set, const u32x4 (&ra)[AI][2], const u32x4 (&rb)[BI][2]) {
        uint16_t *sa = smem + buf * STAGE;
        uint16_t *sb = sa + BMK * LDK;
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int it = tid + NT * j, p = item_p(it), cc = item_c(it);
            u32x4 d[2] = {ra[j][0], ra[j][1]};
            if constexpr (FUSE) {
                float mu[8], is[8], ca[8], cb[8], cg[8];
                bnbwd_coef8(sbn, BMK, 8 * cc, mu, is, ca, cb, cg);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 v = bnbwd_dz8(ra[j][h], rz2[set][j][h], rm2[set][j][h], mu, is, ca, cb, cg);
                    d[h] = ((okm2[set] >> (2 * j + h)) & 1u) ? v : u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t lo = (d[0][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                const uint32_t hi = (d[1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                *(uint32_t *)(sa + swz(8 * cc + e, 2 * p)) = lo | (hi << 16);
            }
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const int it = tid + NT * j, p = item_p(it), cc = item_c(it);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t lo = (rb[j][0][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                const uint32_t hi = (rb[j][1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                *(uint32_t *)(sb + swz(8 * cc + e, 2 * p)) = lo | (hi << 16);
            }
        }
    };

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // 32x32x16 fragments: lane l reads row (l & 31), pixels 8*(l >> 5)..+7 of slice kh;
    // the fragments of slice kh + 1 are read while the MFMAs of slice kh run.
    auto compute = [&](int buf) {
        const uint16_t *sa = smem + buf * STAGE;
        const uint16_t *sb = sa + BMK * LDK;
        bf16x8 a[2][MI], b[2][NJ];
        auto rd = [&](int kh, int d) {
            const int mb = kh * 16 + (lane >> 5) * 8;
#pragma unroll
            for (int i = 0; i < MI; ++i) a[d][i] = *(const bf16x8 *)(sa + swz(wm * WM + 32 * i + (lane & 31), mb));
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[d][j] = *(const bf16x8 *)(sb + swz(wn * WN + 32 * j + (lane & 31), mb));
        };
        rd(0, 0);
#pragma unroll
        for (int kh = 0; kh < BKM / 16; ++kh) {
            if (kh + 1 < BKM / 16) rd(kh + 1, (kh + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kh & 1][i], b[kh & 1][j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int nsteps = (mend - mbeg + BKM - 1) / BKM;
    if constexpr (STAGES == 2) {
        // Two register stages: the loads of a K-step are issued two K-steps ahead.
        u32x4 ra2[2][AI][2], rb2[2][BI][2];
        if (nsteps > 0) {
            load(mbeg, 0, ra2[0], rb2[0]);
            if (nsteps > 1) load(mbeg + BKM, 1, ra2[1], rb2[1]);
            store(0, 0, ra2[0], rb2[0]);
        }
        __syncthreads();
        for (int st = 0; st < nsteps; st += 2) {
            if (st + 2 < nsteps) load(mbeg + (st + 2) * BKM, 0, ra2[0], rb2[0]);
            compute(0);
            if (st + 1 < nsteps) store(1, 1, ra2[1], rb2[1]);
            __syncthreads();
            if (st + 1 >= nsteps) break;
            if (st + 3 < nsteps) load(mbeg + (st + 3) * BKM, 1, ra2[1], rb2[1]);
            compute(1);
            if (st + 2 < nsteps) store(0, 0, ra2[0], rb2[0]);
            __syncthreads();
        }
    } else {
        // One register stage: the loads of a K-step are issued one K-step ahead.
        u32x4 ra[AI][2], rb[BI][2];
        if (nsteps > 0) {
            load(mbeg, 0, ra, rb);
            store(0, 0, ra, rb);
        }
        __syncthreads();
        for (int st = 0; st < nsteps; ++st) {
            const int cur = st & 1;
            if (st + 1 < nsteps) load(mbeg + (st + 1) * BKM, 0, ra, rb);
            compute(cur);
            if (st + 1 < nsteps) store(cur ^ 1, 0, ra, rb);
            __syncthreads();
        }
    }

    // Accumulator layout of v_mfma_f32_32x32x16: lane l holds column (l & 31) and rows
    // 8*(v/4) + 4*(l >> 5) + v%4 of each 32 x 32 block.
    float *out = prm.out + (size_t)blockIdx.z * g.K * g.Kg;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int k = k0 + wm * WM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int kk = n0 + wn * WN + 32 * j + (lane & 31);
                if (k < g.K && kk < g.Kg) out[(size_t)k * g.Kg + kk] = acc[i][j][v];
            }
}

// dw[i] = sum over splits s (in order) of part[s][i].  n % 4 == 0 takes 16-byte loads,
// every split's load of a thread in flight at once.
__global__ __launch_bounds__(NT) void split_sum_kernel(const float *__restrict__ part, int splits, long n,
                                                       float *__restrict__ dw)
{
    if ((n & 3) == 0) {
        const long n4 = n >> 2;
        const f32x4 *p4 = (const f32x4 *)part;
        for (long i = (long)blockIdx.x * NT + threadIdx.x; i < n4; i += (long)gridDim.x * NT) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            int t = 0;
            for (; t + 4 <= splits; t += 4) {
                const f32x4 a = p4[(size_t)t * n4 + i], b = p4[(size_t)(t + 1) * n4 + i];
                const f32x4 c = p4[(size_t)(t + 2) * n4 + i], d = p4[(size_t)(t + 3) * n4 + i];
                s += a;
                s += b;
                s += c;
                s += d;
            }
            for (; t < splits; ++t) s += p4[(size_t)t * n4 + i];
            ((f32x4 *)dw)[i] = s;
        }
        return;
    }
    for (long i = (long)blockIdx.x * NT + threadIdx.x; i < n; i += (long)gridDim.x * NT) {
        float s = 0.f;
        for (int t = 0; t < splits; ++t) s += part[(size_t)t * n + i];
        dw[i] = s;
    }
}

// Filter of the data gradient as a forward convolution (stride 1):
// wt[c][r'][s'][k] = w[k][R-1-r'][S-1-s'][c].  Thread t makes the eight outputs of
// k = 8 k8 .. 8 k8 + 7 at one (c, r', s'), t = ((k8 R + r') S + s') C + c: its eight
// 2-byte reads are coalesced over the threads of consecutive c, and the outputs leave as
// one 16-byte store (K % 8 == 0).  32-bit indices: filters hold far fewer than 2^31
// elements.
__global__ __launch_bounds__(NT) void flip_weights_kernel(const uint16_t *__restrict__ w, int K, int R, int S, int C,
                                                          uint16_t *__restrict__ wt)
{
    const int total = (K / 8) * R * S * C;
    const int rsc = R * S * C;
    for (int t = blockIdx.x * NT + threadIdx.x; t < total; t += gridDim.x * NT) {
        const int c = t % C;
        int u = t / C;
        const int s = u % S;
        u /= S;
        const int r = u % R, k8 = u / R;
        const uint16_t *src = w + ((size_t)(8 * k8) * R + (R - 1 - r)) * S * C + (S - 1 - s) * C + c;
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (uint32_t)src[(size_t)(2 * e) * rsc] | ((uint32_t)src[(size_t)(2 * e + 1) * rsc] << 16);
        *(u32x4 *)(wt + (((size_t)c * R + r) * S + s) * K + 8 * k8) = u32x4{v[0], v[1], v[2], v[3]};
    }
}


// ---------------------------------------------------------------------------------
// Transposed-read form (C % 128 == 0, K % 256 == 0): dz and im2col(x) slices are moved
// into LDS unchanged (pixel rows, channels contiguous) by buffer-to-LDS loads, and the
// MFMA fragments -- 8 consecutive pixels of one channel per lane -- come out of LDS with
// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4a + b receives element b of the
// 8-byte rows addressed by lanes a, a + 4, a + 8 and a + 12.  Lane i of a group therefore
// addresses pixel (i / 4) at channel 4 (i % 4) of its 16-channel group, and lane 4a + b
// ends up with channel 4a + b of four consecutive pixels; two such reads make one
// fragment.  Rows are 512 (dz) or 256 (x) bytes; the 64-byte unit u of pixel row m sits
// at unit u ^ (m % 4), so the four pixel rows of a read hit distinct banks.
// The workgroup tile is 256 output channels x 128 filter positions (one tap, 128 input
// channels), eight waves in a 4 x 2 grid of 64 x 64 wave tiles; the pixel range is split
// over the grid's second dimension.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

struct WgradTrParams {
    const uint16_t *dz, *x;
    float *out;            // [splits][K][Kg] (dw itself when splits == 1)
    int N, H, W, C, K, S, sh, sw, ph, pw, P, Q, M, Kg;
    int rows_per_split;
    FastDiv dpq, dq;
};

__device__ __forceinline__ i16x4 lds_tr16(uint32_t addr)
{
    i16x4 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
template <int N>
__device__ __forceinline__ void tr_lgkm_wait() { asm volatile("s_waitcnt lgkmcnt(%0)" : : "i"(N) : "memory"); }
template <int N>
__device__ __forceinline__ void tr_vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory"); }
__device__ __forceinline__ void tr_tie(i16x4 &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void tr_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    tr_lgkm_wait<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}
// (A device function: the builtin has no host form.)
__device__ __forceinline__ void tr_buffer_load_lds16(__amdgpu_buffer_rsrc_t r, lds_u8 *dst, int voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 tr_join(i16x4 lo, i16x4 hi)
{
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Tile configurations: BM output channels x BN filter positions (one tap, BN input
// channels) per workgroup, WGM x WGN waves, NSTAGE slices of 64 pixels in LDS.
template <int BM_, int BN_, int WGM_, int WGN_, int NSTAGE_>
struct TrCfg {
    static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, NSTAGE = NSTAGE_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int BKM = 64;                              // pixels per slice
    static constexpr int RSA = 2 * BM, RSB = 2 * BN;            // row bytes of the dz and x slices
    static constexpr int STAGE_A = BKM * RSA, STAGE = STAGE_A + BKM * RSB;
    static constexpr int NA = STAGE_A / 1024, NINS = STAGE / 1024;   // 1 KB load instructions
    static constexpr int IPW = NINS / NW;
    static constexpr size_t LDS = (size_t)NSTAGE * STAGE;
    static_assert(NINS % NW == 0 && NA % NW == 0, "load instructions per wave");
    static_assert(NSTAGE == 2 || NSTAGE == 3, "slices in LDS");
};
// 256 x 128 tiles, eight 64 x 64 wave tiles, three slices in flight (PLAN_WG_TR), and
// 256 x 256 tiles, eight 128 x 64 wave tiles (a quarter fewer fragment bytes per MFMA),
// two slices (PLAN_WG_TR_WIDE).
using TrStd = TrCfg<256, 128, 4, 2, 3>;
using TrWide = TrCfg<256, 256, 2, 4, 2>;

template <typename C>
__global__ __launch_bounds__(C::NT, 1) void conv_wgrad_tr_kernel(WgradTrParams p)
{
    constexpr int TR_BM = C::BM, TR_BN = C::BN, TR_WGM = C::WGM, TR_WGN = C::WGN, TR_NSTAGE = C::NSTAGE;
    constexpr int TR_NW = C::NW, TR_BKM = C::BKM, TR_RSA = C::RSA, TR_RSB = C::RSB;
    constexpr int TR_STAGE_A = C::STAGE_A, TR_STAGE = C::STAGE, TR_NA = C::NA, TR_IPW = C::IPW;
    constexpr int MI = TR_BM / (32 * TR_WGM), NJ = TR_BN / (32 * TR_WGN);   // blocks per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_u8 *)lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / TR_WGN, wn = wave % TR_WGN;
    const int k0 = blockIdx.y * TR_BM, kk0 = blockIdx.x * TR_BN;
    const int tap = kk0 / p.C, c0 = kk0 - tap * p.C;
    const int tr = tap / p.S, ts = tap - tr * p.S;
    const int m0 = blockIdx.z * p.rows_per_split;
    const int m1 = min(p.M, m0 + p.rows_per_split);
    const int nsteps = m1 > m0 ? (m1 - m0 + TR_BKM - 1) / TR_BKM : 0;
    const __amdgpu_buffer_rsrc_t dzr =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.dz, 0, 2 * p.M * p.K, 0x00020000);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.x, 0, 2 * p.N * p.H * p.W * p.C, 0x00020000);

    // Slice loads of pixels mb .. mb + 63 into stage st: instruction u (wave u % NW) moves
    // 1 KB of rows; lane l the 16 bytes at byte 16 l of it.  Instructions q < ZQ of a
    // wave are dz rows, the others x rows.  A lane's pixel in an instruction advances by
    // 64 per slice, so its decode (n, p, q) and x offset are kept per instruction and
    // stepped with adds (64 = sa * Q + sb); multiply-high divisions per slice cost more
    // than the loads themselves.
    constexpr int ZQ = TR_NA / TR_NW;              // dz instructions per wave
    constexpr int XQ = TR_IPW - ZQ;                // x instructions per wave
    static_assert(TR_NA % TR_NW == 0, "dz and x instructions split per wave");
    int zoff[ZQ];                                  // dz byte offset of the lane's row, current slice
    int xm[XQ], xn[XQ], xp[XQ], xq[XQ], xoff[XQ];  // x row: pixel, its (n, p, q), byte offset
    const int sa = TR_BKM / p.Q, sb = TR_BKM - sa * p.Q;
#pragma unroll
    for (int q = 0; q < ZQ; ++q) {
        const int u = wave + TR_NW * q;
        const int row = u * (1024 / TR_RSA) + (16 * lane) / TR_RSA;
        const int b = (16 * lane) % TR_RSA;
        zoff[q] = 2 * ((m0 + row) * p.K + k0) + (b ^ ((row & 3) << 6));
    }
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
        const int u = wave + TR_NW * (ZQ + q);
        const int row = (u - TR_NA) * (1024 / TR_RSB) + (16 * lane) / TR_RSB;
        const int b = (16 * lane) % TR_RSB;
        const int m = m0 + row;
        xm[q] = m;
        xn[q] = (int)div_by((uint32_t)m, p.dpq);
        const int rem = m - xn[q] * p.P * p.Q;
        xp[q] = (int)div_by((uint32_t)rem, p.dq);
        xq[q] = rem - xp[q] * p.Q;
        xoff[q] = 2 * (((xn[q] * p.H + xp[q] * p.sh - p.ph + tr) * p.W + xq[q] * p.sw - p.pw + ts) * p.C + c0) +
                  (b ^ ((row & 3) << 6));
    }
    // x offset steps: one column, one row wrap, one image wrap
    const int dcol = 2 * p.sw * p.C, drow = 2 * (p.sh * p.W - p.Q * p.sw) * p.C;
    const int dimg = 2 * (p.H - p.P * p.sh) * p.W * p.C;
    auto dma_issue = [&](int t) __attribute__((always_inline)) {
        const uint32_t st = (uint32_t)((t % TR_NSTAGE) * TR_STAGE);
#pragma unroll
        for (int q = 0; q < ZQ; ++q) {
            const int u = wave + TR_NW * q;
            const int m = m0 + t * TR_BKM + u * (1024 / TR_RSA) + (16 * lane) / TR_RSA;
            tr_buffer_load_lds16(dzr, (lds_u8 *)lds + st + u * 1024, m < m1 ? zoff[q] : (int)OOB);
            zoff[q] += 2 * TR_BKM * p.K;
        }
#pragma unroll
        for (int q = 0; q < XQ; ++q) {
            const int u = wave + TR_NW * (ZQ + q);
            const int h = xp[q] * p.sh - p.ph + tr, w = xq[q] * p.sw - p.pw + ts;
            const bool ok = xm[q] < m1 && (unsigned)h < (unsigned)p.H && (unsigned)w < (unsigned)p.W;
            tr_buffer_load_lds16(xr, (lds_u8 *)lds + st + u * 1024, ok ? xoff[q] : (int)OOB);
            // advance the pixel by 64: sa rows and sb columns, with wraps
            xm[q] += TR_BKM;
            xq[q] += sb;
            xp[q] += sa;
            xoff[q] += sb * dcol + sa * (drow + p.Q * dcol);
            if (xq[q] >= p.Q) {
                xq[q] -= p.Q;
                ++xp[q];
                xoff[q] += drow;
            }
            while (xp[q] >= p.P) {
                xp[q] -= p.P;
                ++xn[q];
                xoff[q] += dimg;
            }
        }
    };
    // Fragment addresses: lane l of group G = l / 16, i = l % 16 reads pixel
    // 16 kh + 8 (G / 2) + 4 r + i / 4 at channel 16 (G % 2) + 4 (i % 4) of its block.
    const int G = lane >> 4, li = lane & 15;
    const int prow = 8 * (G >> 1) + (li >> 2);
    uint32_t aa[MI], ba[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int byte = 2 * (wm * 32 * MI + 32 * i + 16 * (G & 1) + 4 * (li & 3));
        aa[i] = lbase + prow * TR_RSA + (byte ^ ((prow & 3) << 6));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int byte = 2 * (wn * 32 * NJ + 32 * j + 16 * (G & 1) + 4 * (li & 3));
        ba[j] = lbase + TR_STAGE_A + prow * TR_RSB + (byte ^ ((prow & 3) << 6));
    }
    i16x4 af[3][MI][2], bf[3][NJ][2];
    auto read_frags = [&](i16x4 (&a)[MI][2], i16x4 (&b)[NJ][2], int t, int kh) __attribute__((always_inline)) {
        const uint32_t so = (uint32_t)((t % TR_NSTAGE) * TR_STAGE);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            a[i][0] = lds_tr16(aa[i] + so + (16 * kh) * TR_RSA);
            a[i][1] = lds_tr16(aa[i] + so + (16 * kh + 4) * TR_RSA);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            b[j][0] = lds_tr16(ba[j] + so + (16 * kh) * TR_RSB);
            b[j][1] = lds_tr16(ba[j] + so + (16 * kh + 4) * TR_RSB);
        }
    };
    constexpr int NRD = 2 * (MI + NJ);   // reads per fragment set

    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    auto mfma = [&](const i16x4 (&a)[MI][2], const i16x4 (&b)[NJ][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_join(a[i][0], a[i][1]), tr_join(b[j][0], b[j][1]),
                                                                    acc[i][j], 0, 0, 0);
    };
    auto tie_set = [&](i16x4 (&a)[MI][2], i16x4 (&b)[NJ][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i) { tr_tie(a[i][0]); tr_tie(a[i][1]); }
#pragma unroll
        for (int j = 0; j < NJ; ++j) { tr_tie(b[j][0]); tr_tie(b[j][1]); }
    };

    if constexpr (TR_NSTAGE == 3) {
        // Three slices in LDS, the barrier in mid-slice (after k-step 1), fragment sets read
        // two k-steps ahead, three sets rotating (k-step kh of slice t uses set (4t + kh) % 3).
        // The mid-slice barrier of slice t publishes slice t + 1 (each wave waits for its own
        // loads of it first) and shows every wave past slice t - 1, whose buffer then takes
        // slice t + 2's loads.  Slice t + 1's first two fragment sets are read during k-steps
        // 2 and 3 of slice t, so no k-step waits behind a barrier for its reads.
        const int npro = min(2, nsteps);
        for (int t = 0; t < npro; ++t) dma_issue(t);
        if (nsteps > 0) {
            if (npro > 1) tr_vm_wait<TR_IPW>();
            else tr_vm_wait<0>();
            tr_barrier();
            read_frags(af[0], bf[0], 0, 0);
            read_frags(af[1], bf[1], 0, 1);
        }
        auto slice = [&](int t, auto pc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;
            constexpr int S0 = P % 3, S1 = (P + 1) % 3, S2 = (P + 2) % 3;   // k-step 3 uses S0 again
            const bool more = t + 1 < nsteps;
            // k-step 0
            tr_lgkm_wait<NRD>();
            tie_set(af[S0], bf[S0]);
            __builtin_amdgcn_sched_barrier(0);
            mfma(af[S0], bf[S0]);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(af[S2], bf[S2], t, 2);
            // k-step 1
            tr_lgkm_wait<NRD>();
            tie_set(af[S1], bf[S1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma(af[S1], bf[S1]);
            __builtin_amdgcn_sched_barrier(0);
            read_frags(af[S0], bf[S0], t, 3);
            // mid-slice barrier (no LDS wait: the reads in flight are of slice t, and every
            // read of slice t - 1 was waited for at its own k-steps)
            if (more) tr_vm_wait<0>();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (t + 2 < nsteps) dma_issue(t + 2);
            __builtin_amdgcn_sched_barrier(0);
            // k-step 2
            tr_lgkm_wait<NRD>();
            tie_set(af[S2], bf[S2]);
            __builtin_amdgcn_sched_barrier(0);
            mfma(af[S2], bf[S2]);
            __builtin_amdgcn_sched_barrier(0);
            if (more) read_frags(af[S1], bf[S1], t + 1, 0);
            // k-step 3
            if (more) tr_lgkm_wait<NRD>();
            else tr_lgkm_wait<0>();
            tie_set(af[S0], bf[S0]);
            __builtin_amdgcn_sched_barrier(0);
            mfma(af[S0], bf[S0]);
            __builtin_amdgcn_sched_barrier(0);
            if (more) read_frags(af[S2], bf[S2], t + 1, 1);
        };
        for (int t = 0; t < nsteps; t += 3) {
            slice(t, std::integral_constant<int, 0>{});
            if (t + 1 < nsteps) slice(t + 1, std::integral_constant<int, 1>{});
            if (t + 2 < nsteps) slice(t + 2, std::integral_constant<int, 2>{});
        }
    } else {
        // Slice t lives in stage t % 3; slices t + 1 and t + 2 are in flight while it is used.
        const int npro = min(TR_NSTAGE - 1, nsteps);
        for (int t = 0; t < npro; ++t) dma_issue(t);
        if (nsteps > 0) {
            if (npro > 1) tr_vm_wait<TR_IPW>();
            else tr_vm_wait<0>();
            tr_barrier();
            read_frags(af[0], bf[0], 0, 0);
        }
        for (int t = 0; t < nsteps; ++t) {
    #pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
                read_frags(af[(kh + 1) & 1], bf[(kh + 1) & 1], t, kh + 1);
                tr_lgkm_wait<NRD>();
                tie_set(af[kh & 1], bf[kh & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mfma(af[kh & 1], bf[kh & 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (kh == 0 && t + TR_NSTAGE - 1 < nsteps) dma_issue(t + TR_NSTAGE - 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            tr_lgkm_wait<0>();
            tie_set(af[1], bf[1]);
            // slice t + 1 landed (with three stages slice t + 2 may stay in flight); every wave
            // is past slice t
            if constexpr (TR_NSTAGE == 3) {
                if (t + 2 < nsteps) tr_vm_wait<TR_IPW>();
                else if (t + 1 < nsteps) tr_vm_wait<0>();
            } else {
                if (t + 1 < nsteps) tr_vm_wait<0>();
            }
            tr_barrier();
            if (t + 1 < nsteps) read_frags(af[0], bf[0], t + 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            mfma(af[1], bf[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Accumulator layout of v_mfma_f32_32x32x16: lane l holds column (l & 31) and rows
    // 8*(v/4) + 4*(l >> 5) + v%4 of each 32 x 32 block.
    float *out = p.out + (size_t)blockIdx.z * p.K * p.Kg;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int k = k0 + wm * 32 * MI + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int kk = kk0 + wn * 32 * NJ + 32 * j + (lane & 31);
                out[(size_t)k * p.Kg + kk] = acc[i][j][v];
            }
}

}  // namespace

bool wgrad_tr_eligible(const ConvGeom &g, int bn)
{
    const double xbytes = 2.0 * g.N * g.H * g.W * g.C, zbytes = 2.0 * g.M * g.K;
    return g.C % bn == 0 && g.K % TrStd::BM == 0 && g.M > 0 && xbytes < 2147483648.0 && zbytes < 2147483648.0;
}
bool wgrad_tr_eligible(const ConvGeom &g) { return wgrad_tr_eligible(g, TrStd::BN); }
bool wgrad_tr_wide_eligible(const ConvGeom &g) { return wgrad_tr_eligible(g, TrWide::BN); }

WgradPlan wgrad_plan(const ConvGeom &g, int plan)
{
    const int M = g.M, K = g.K, Kg = g.Kg;
    WgradPlan p;
    p.tr = plan == PLAN_WG_TR || plan == PLAN_WG_TR_WIDE;
    if (p.tr) {
        // one workgroup per CU: 256 x 128 (or 256 x 256) tiles, the pixel range split to
        // fill the rest
        p.bm = TrStd::BM;
        p.bn = plan == PLAN_WG_TR_WIDE ? TrWide::BN : TrStd::BN;
        p.tiles_m = K / p.bm;
        p.tiles_n = Kg / p.bn;
        const int tiles = p.tiles_m * p.tiles_n;
        const int steps = (M + TrStd::BKM - 1) / TrStd::BKM;
        const int want = std::max(1, std::min(steps, 256 / tiles));
        const int steps_per = (steps + want - 1) / want;
        p.rows_per_split = steps_per * TrStd::BKM;
        p.splits = (M + p.rows_per_split - 1) / p.rows_per_split;
        return p;
    }
    p.bm = K >= 128 ? 128 : 64;
    p.bn = 128;
    p.tiles_m = (K + p.bm - 1) / p.bm;
    p.tiles_n = (Kg + p.bn - 1) / p.bn;
    const int tiles = p.tiles_m * p.tiles_n;
    int want = std::max(1, std::min(256, (512 + tiles - 1) / tiles));
    const int steps = (M + BKM - 1) / BKM;
    want = std::min(want, steps);
    const int steps_per = (steps + want - 1) / want;
    p.rows_per_split = steps_per * BKM;
    p.splits = (M + p.rows_per_split - 1) / p.rows_per_split;
    return p;
}

// The generic weight-gradient kernel for plan p, then the fixed-order split sum.
template <bool FUSE>
hipError_t launch_wgrad_generic(const ConvGeom &g, const WgradPlan &p, const WgradParams &prm, float *part, float *dw,
                                hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    dim3 grid(p.tiles_n, p.tiles_m, p.splits);
    const bool vec = (g.C % 8) == 0;
    const hipEvent_t ek = p.splits == 1 ? e1 : nullptr;   // end event on the last kernel of the stage
    hipError_t e;
    if constexpr (FUSE) {   // C % 8 == 0 (the fused plan's condition): 16-byte gathers of x
        e = p.bm == 128 ? launch(conv_wgrad_kernel<128, 128, true, WGRAD_STAGES_128, true>, grid, dim3(NT), 0, st, e0,
                                 ek, prm)
                        : launch(conv_wgrad_kernel<64, 128, true, 2, true>, grid, dim3(NT), 0, st, e0, ek, prm);
    } else if (p.bm == 128) {
        e = vec ? launch(conv_wgrad_kernel<128, 128, true, WGRAD_STAGES_128>, grid, dim3(NT), 0, st, e0, ek, prm)
                : launch(conv_wgrad_kernel<128, 128, false, 1>, grid, dim3(NT), 0, st, e0, ek, prm);
    } else {
        e = vec ? launch(conv_wgrad_kernel<64, 128, true, 2>, grid, dim3(NT), 0, st, e0, ek, prm)
                : launch(conv_wgrad_kernel<64, 128, false, 1>, grid, dim3(NT), 0, st, e0, ek, prm);
    }
    if (e != hipSuccess || p.splits == 1) return e;
    const long n = (long)g.K * g.Kg;
    const int blocks = (int)std::min<long>((n + NT - 1) / NT, 8192);
    return launch(split_sum_kernel, dim3(blocks), dim3(NT), 0, st, nullptr, e1, (const float *)part, p.splits, n, dw);
}

// Whether the split partials of plan p fit a buffer of part_bytes.
bool parts_fit(const ConvGeom &g, const WgradPlan &p, size_t part_bytes)
{
    return p.splits <= 1 || sizeof(float) * (size_t)p.splits * g.K * g.Kg <= part_bytes;
}

hipError_t launch_conv_wgrad(const ConvGeom &g, int plan, const uint16_t *dz, const uint16_t *x, float *part,
                             size_t part_bytes, float *dw, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    const WgradPlan p = wgrad_plan(g, plan);
    if (!parts_fit(g, p, part_bytes)) return hipErrorInvalidValue;
    if (p.tr) {
        WgradTrParams tp;
        tp.dz = dz;
        tp.x = x;
        tp.out = p.splits == 1 ? dw : part;
        tp.N = g.N; tp.H = g.H; tp.W = g.W; tp.C = g.C; tp.K = g.K; tp.S = g.S;
        tp.sh = g.sh; tp.sw = g.sw; tp.ph = g.ph; tp.pw = g.pw; tp.P = g.P; tp.Q = g.Q; tp.M = g.M; tp.Kg = g.Kg;
        tp.rows_per_split = p.rows_per_split;
        tp.dpq = fast_div((uint32_t)(g.P * g.Q));
        tp.dq = fast_div((uint32_t)g.Q);
        const hipEvent_t ek = p.splits == 1 ? e1 : nullptr;
        auto run = [&](auto cfg) {
            using C = decltype(cfg);
            hipError_t e = raise_lds_limit((const void *)conv_wgrad_tr_kernel<C>, (int)C::LDS);
            if (e != hipSuccess) return e;
            return launch(conv_wgrad_tr_kernel<C>, dim3(p.tiles_n, p.tiles_m, p.splits), dim3(C::NT),
                          (uint32_t)C::LDS, st, e0, ek, tp);
        };
        const hipError_t e = p.bn == TrWide::BN ? run(TrWide{}) : run(TrStd{});
        if (e != hipSuccess || p.splits == 1) return e;
        const long n = (long)g.K * g.Kg;
        const int blocks = (int)std::min<long>((n + NT - 1) / NT, 8192);
        return launch(split_sum_kernel, dim3(blocks), dim3(NT), 0, st, nullptr, e1, (const float *)part, p.splits, n,
                      dw);
    }
    WgradParams prm{g,       dz,      x,       p.splits == 1 ? dw : part, p.rows_per_split, fast_div((uint32_t)(g.P * g.Q)),
                    fast_div((uint32_t)g.Q), nullptr, nullptr, nullptr, nullptr};
    return launch_wgrad_generic<false>(g, p, prm, part, dw, st, e0, e1);
}

hipError_t launch_conv_wgrad_fused(const ConvGeom &g, const uint16_t *dy, const uint16_t *z, const uint8_t *mask,
                                   const float *bnc, const uint16_t *x, float *part, size_t part_bytes, float *dw,
                                   hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    const WgradPlan p = wgrad_plan(g, PLAN_WG_GEN);
    if (!parts_fit(g, p, part_bytes)) return hipErrorInvalidValue;
    WgradParams prm{g,       nullptr, x,  p.splits == 1 ? dw : part, p.rows_per_split, fast_div((uint32_t)(g.P * g.Q)),
                    fast_div((uint32_t)g.Q), dy, z,  mask, bnc};
    return launch_wgrad_generic<true>(g, p, prm, part, dw, st, e0, e1);
}

hipError_t launch_flip_weights(int K, int R, int S, int C, const uint16_t *w, uint16_t *wt, hipStream_t st,
                               hipEvent_t e0, hipEvent_t e1)
{
    const long total = (long)(K / 8) * R * S * C;   // K % 8 == 0 (shape validation)
    const int blocks = (int)std::min<long>((total + NT - 1) / NT, 4096);
    return launch(flip_weights_kernel, dim3(blocks), dim3(NT), 0, st, e0, e1, w, K, R, S, C, wt);
}

}  // namespace cbr
