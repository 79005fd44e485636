// conv_igemm.hip -- persistent large-tile implicit-GEMM convolution for C % 32 == 0.
//
// GEMM view as in conv_fprop.hip: rows are output pixels m = (n,p,q), columns output
// channels k, reduction over kk = (r,s,c), c fastest.  Differences, all aimed at keeping
// the matrix cores fed on the larger layers:
//   * At most 256 workgroups (one per CU), each owning a contiguous range of output
//     pixels that it walks in chunks of BM pixels x BN channels.  A short last chunk
//     skips the MFMAs of pixel blocks that hold no pixel, so the ragged tail of an
//     uneven M costs its own size, not a whole tile.
//   * WGM x WGN waves, each with a wave tile of MI pixel blocks x NJ channel blocks of 32
//     (v_mfma_f32_32x32x16_bf16, the filter as the A operand, so a lane's results are
//     four consecutive channels of one pixel).  Large wave tiles keep the LDS fragment
//     reads per MFMA low.
//   * Reduction slices of BK = 64 (C % 64 == 0) or 32 elements, inside one filter tap,
//     taken channel slice by channel slice, all taps of one before the next (the rows the
//     taps re-read are then BK channels wide instead of C, a smaller set for the XCD's L2
//     to hold), move from global memory straight into LDS (buffer-to-LDS loads, 128- or 64-byte
//     rows, 16-byte chunks XOR-permuted by row so fragment reads are conflict-free),
//     NSTAGE slices in flight.
//     Padding taps and pixels past the range get out-of-range buffer offsets (zeros).  The slice
//     sequence runs on across chunk boundaries, so a chunk's epilogue overlaps the next
//     chunk's first loads.
//   * Results leave through an LDS staging tile as whole 16-byte chunks of contiguous
//     output rows.
// Epilogues as in conv_fprop.hip: EPI_STATS (z + per-channel count, mean and M2 of each
// pixel chunk's fp32 accumulators, two passes over the registers: the CBR page's conv +
// genstats, section 4.1), EPI_BIAS_RELU (the folded-BN inference form, CBR page sections
// 2 and 6, and the TileLang page's Conv2D + ReLU), EPI_PLAIN (data gradient), EPI_BIAS
// (Conv2D + bias).  A NULL bias reads as zeros.
#include <type_traits>

#include "cbr_launch.h"

namespace cbr {
namespace {


typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

struct IgParams {
    const uint16_t *x, *w;
    const float *bias;
    uint16_t *out;
    float *partials;
    int N, H, W, C, K, R, S;
    int sh, sw, ph, pw;
    int P, Q, M, Kg;
    int ksteps;        // Kg / BK slices per chunk
    int rows_per_wg;   // contiguous output pixels per workgroup
    int ntn;           // K / BN
    int maxmc;         // pixel chunks per workgroup at most (statistics rows per workgroup)
};

constexpr uint32_t OOB = 0x80000000u;   // past the end of every buffer (sizes < 2^31)


// LDS accesses in inline assembly.  With global-to-LDS loads in flight the compiler
// waits for all of them before any LDS access it emits itself; these are outside its
// tracking, and the kernel waits for exactly what each access needs.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr)
{
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}
__device__ __forceinline__ u32x4 lds_read16u(uint32_t addr)
{
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ void lds_write8(uint32_t addr, u32x2 v)
{
    asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
template <int N>
__device__ __forceinline__ void lgkm_wait() { asm volatile("s_waitcnt lgkmcnt(%0)" : : "i"(N) : "memory"); }
template <int N>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory"); }
// 16 bytes per lane from buffer offset voff to LDS dst + 16 * lane (zeros past the end).
// (A device function: the builtin has no host form, and in a kernel body it would keep
// the kernel's host-side stub from being emitted.)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, lds_u8 *dst, int voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

// N fragments at base + i * STRIDE (immediate offsets).
template <int I, int N, int STRIDE>
__device__ __forceinline__ void read_frag_row(bf16x8 (&f)[N], uint32_t base)
{
    if constexpr (I < N) {
        f[I] = lds_read16<I * STRIDE>(base);
        read_frag_row<I + 1, N, STRIDE>(f, base);
    }
}

// The MFMAs of one fragment set on the first NB pixel blocks: acc[i][j] += A(filter j) *
// B(pixels i).  NB is a template argument so the MFMA sequence has no branches: a branch
// per block makes the compiler move the accumulators between register files each time.
template <int MI, int NJ, int NB>
__device__ __forceinline__ void mfma_set(f32x16 (&acc)[MI][NJ], const bf16x8 (&a)[NJ], const bf16x8 (&b)[MI])
{
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[i], acc[i][j], 0, 0, 0);
}

// Ties a register to the preceding wait, so its use cannot be scheduled above it.
__device__ __forceinline__ void after_wait(bf16x8 &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void after_wait(u32x4 &x) { asm volatile("" : "+v"(x)); }

// Workgroup barrier; the wave's own LDS accesses complete first (s_barrier alone does
// not wait for them).  Global-to-LDS loads are waited for separately (vmcnt).
__device__ __forceinline__ void barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    lgkm_wait<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// vmcnt wait for "at most n * PER outstanding", n < 4 at run time.
template <int PER>
__device__ __forceinline__ void vm_wait_steps(int n)
{
    if (n >= 3) vm_wait<3 * PER>();
    else if (n == 2) vm_wait<2 * PER>();
    else if (n == 1) vm_wait<PER>();
    else vm_wait<0>();
}

// MI, NJ: pixel / channel blocks of 32 per wave; WGM x WGN waves per workgroup; BK
// reduction elements per slice, NSTAGE slices in flight.  The epilogue stages the output
// tile (and the statistics) in the slice buffers, so a chunk's loads stop at its end.
template <int MI, int NJ, int WGM, int WGN, int BK, int NSTAGE, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void conv_igemm_kernel(IgParams p)
{
    constexpr int NW = WGM * WGN, NT = 64 * NW;
    constexpr int BM = 32 * MI * WGM, BN = 32 * NJ * WGN;
    constexpr int RB = 2 * BK;                    // bytes per staged row
    constexpr int CPR = RB / 16;                  // 16-byte chunks per row
    constexpr int RPI = 1024 / RB;                // rows per 1 KB load instruction
    constexpr int KH = BK / 16;                   // MFMA k-steps per slice
    constexpr int ROWS = BM + BN;                 // staged rows per slice
    constexpr int NINS = ROWS / RPI;              // load instructions per slice
    constexpr int IPW = (NINS + NW - 1) / NW;     // per wave, at most
    constexpr int LMIN = NINS / NW;               // per wave, at least
    constexpr int STAGE_B = ROWS * RB;
    constexpr int STG_ROW = 2 * BN;               // staging bytes per pixel
    constexpr int NF = NJ * 32;                   // statistics values per lane
    constexpr int SCR_B = EPI == EPI_STATS ? NW * 64 * NF * 4 : 0;   // statistics scratch
    static_assert(BN >= 128 && BM % 32 == 0 && (BK == 32 || BK == 64), "tile shape");
    static_assert(NSTAGE * STAGE_B >= BM * STG_ROW && NSTAGE * STAGE_B >= SCR_B,
                  "the epilogue must fit the slice buffers");

    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_u8 *)lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int l32 = lane & 31, hi = lane >> 5;
    const int wm = wave / WGN, wn = wave % WGN;
    float *stat_acc = (float *)(lds + NSTAGE * STAGE_B);

    const int r0 = blockIdx.x * p.rows_per_wg;
    const int r1 = min(p.M, r0 + p.rows_per_wg);
    const int nmc = r1 > r0 ? (r1 - r0 + BM - 1) / BM : 0;
    const int nchunk = nmc * p.ntn;
    const int total = nchunk * p.ksteps;

    // Statistics rows: row blockIdx.x * maxmc + mc holds pixel chunk mc of this workgroup;
    // the rows of chunks it does not have are zeros (count 0).
    float *const counts = p.partials + (size_t)gridDim.x * p.maxmc * 2 * p.K;
    if constexpr (EPI == EPI_STATS) {
        for (int mc = nmc; mc < p.maxmc; ++mc) {
            const int row = blockIdx.x * p.maxmc + mc;
            for (int i = tid; i < 2 * p.K; i += NT) p.partials[(size_t)row * 2 * p.K + i] = 0.f;
            if (tid == 0) counts[row] = 0.f;
        }
    }

    // ---- slice loads: instruction u (rows RPI*u .. RPI*u + RPI - 1) is issued by wave
    // u % NW.  Lane l moves staged row RPI*u + l / CPR, position l % CPR, which holds the
    // row's 16-byte chunk (l % CPR) ^ perm(row), perm(row) = (row / (256 / RB)) % CPR: the
    // 16 rows a fragment read covers then spread over all 64 LDS banks.
    // Buffer resources: a padding tap or a pixel past the range gets an offset past the
    // end, and the load writes zeros to LDS.
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.x, 0, 2 * p.N * p.H * p.W * p.C, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void *)p.w, 0, 2 * p.K * p.Kg, 0x00020000);
    auto perm = [](int row) __attribute__((always_inline)) { return (row / (256 / RB)) % CPR; };
    // Per instruction: d_off = byte offset of the lane's row (pixel rows: of input pixel
    // (n, p*sh - ph, q*sw - pw), channel 0), plus its chunk; d_msk (pixel rows) = bit r of
    // the filter rows and bit 16 + s of the filter columns whose taps fall inside the
    // image (zero for a pixel past the range).
    int d_off[IPW], d_msk[IPW];
    int dchunk = -1, dks = 0, dr = 0, ds = 0, dc0 = 0;
    const int PQ = p.P * p.Q;
    auto dma_chunk = [&](int c) __attribute__((always_inline)) {   // per-lane row data of chunk c
        const int mc = c / p.ntn, n0 = (c - mc * p.ntn) * BN;
        const int cm0 = r0 + mc * BM;
#pragma unroll
        for (int t = 0; t < IPW; ++t) {
            const int u = wave + NW * t;
            const int sr = RPI * u + lane / CPR;
            const int gc16 = ((lane % CPR) ^ perm(sr)) * 16;
            if (u < BM / RPI) {
                const int m = cm0 + sr;
                int msk = 0, off = 0;
                if (m < r1) {
                    const int n = m / PQ, rem = m - n * PQ;
                    const int pp = rem / p.Q, q = rem - pp * p.Q;
                    const int hb = pp * p.sh - p.ph, wb = q * p.sw - p.pw;
                    off = 2 * (((n * p.H + hb) * p.W + wb) * p.C) + gc16;
                    for (int r = 0; r < p.R; ++r) msk |= (unsigned)(hb + r) < (unsigned)p.H ? 1 << r : 0;
                    for (int q2 = 0; q2 < p.S; ++q2) msk |= (unsigned)(wb + q2) < (unsigned)p.W ? 1 << (16 + q2) : 0;
                }
                d_off[t] = off;
                d_msk[t] = msk;
            } else {
                d_off[t] = 2 * (n0 + sr - BM) * p.Kg + gc16;
                d_msk[t] = 0;
            }
        }
    };
    auto dma_issue = [&](int g) __attribute__((always_inline)) {   // slice g (issued in order g = 0, 1, 2, ...)
        if (dks == 0) {
            ++dchunk;
            dma_chunk(dchunk);
            dr = ds = dc0 = 0;
        }
        const uint32_t dst = (uint32_t)((g % NSTAGE) * STAGE_B);
        const int toff = 2 * ((dr * p.W + ds) * p.C + dc0);
        const int koff = 2 * ((dr * p.S + ds) * p.C + dc0);
        const int tapbits = (1 << dr) | (1 << (16 + ds));
#pragma unroll
        for (int t = 0; t < IPW; ++t) {
            const int u = wave + NW * t;
            if (u >= NINS) break;
            if (u < BM / RPI) {
                const bool ok = (d_msk[t] & tapbits) == tapbits;
                buffer_load_lds16(xr, (lds_u8 *)lds + dst + u * 1024, ok ? d_off[t] + toff : (int)OOB);
            } else {
                buffer_load_lds16(wr, (lds_u8 *)lds + dst + u * 1024, d_off[t] + koff);
            }
        }
        // next slice: the next tap of this channel slice, then the next channel slice
        if (++dks == p.ksteps) dks = 0;
        if (++ds == p.S) {
            ds = 0;
            if (++dr == p.R) {
                dr = 0;
                dc0 += BK;
            }
        }
    };

    // ---- fragments ----
    // Filter fragment j: staged row BM + wn*32*NJ + 32j + l32; pixel fragment i: staged
    // row wm*32*MI + 32i + l32; both read chunk 2kh + hi at position (2kh + hi) ^ pa
    // (the row bases are multiples of 32, so perm(row) = perm(l32)).
    const int pa = perm(l32);
    uint32_t fa[KH], xa[KH];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
        const int pos = ((2 * kh + hi) ^ pa) << 4;
        fa[kh] = lbase + (BM + wn * 32 * NJ + l32) * RB + pos;
        xa[kh] = lbase + (wm * 32 * MI + l32) * RB + pos;
    }
    bf16x8 af[2][NJ], bf[2][MI];
    auto read_frags = [&](bf16x8 (&a)[NJ], bf16x8 (&b)[MI], int g, int kh) __attribute__((always_inline)) {
        const uint32_t so = (uint32_t)((g % NSTAGE) * STAGE_B);
        read_frag_row<0, NJ, 32 * RB>(a, fa[kh] + so);
        read_frag_row<0, MI, 32 * RB>(b, xa[kh] + so);
    };

    f32x16 acc[MI][NJ];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    };

    // ---- epilogue of chunk c ----
    auto epilogue = [&](int c) __attribute__((always_inline)) {
        const int mc = c / p.ntn, n0 = (c - mc * p.ntn) * BN;
        const int cm0 = r0 + mc * BM;
        const int nvalid = min(BM, r1 - cm0);
        const uint32_t sbase = lbase;   // the staging tile occupies the slice buffers
        // An opaque copy of the lane id: the addresses below are then computed here, not
        // hoisted out of the main loop and held in registers through it.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int el32 = ln & 31, ehi = ln >> 5;
        if constexpr (EPI == EPI_STATS) {
            // Per channel, over the chunk's nvalid pixels: first the means (per lane over its
            // pixel blocks -- pixels past the range are zeros --, then over the 32 pixel lanes
            // and the WGM pixel-wave rows through LDS), then the squared deviations from
            // them (valid pixels only), reduced the same way.
            float *scr = (float *)lds;
            float *cmean = stat_acc;   // BN channel means of this chunk
            auto reduce = [&](int st, int ch) {
                // ch = wn'*32NJ + 32j + 8(v/4) + 4h + v%4
                const int wn2 = ch / (32 * NJ), cj = ch - wn2 * 32 * NJ;
                const int j = cj >> 5, cr = cj & 31;
                const int v = ((cr >> 3) << 2) | (cr & 3), h = (cr >> 2) & 1;
                float sum = 0.f;
                for (int wm2 = 0; wm2 < WGM; ++wm2) {
                    const float *row = scr + ((wm2 * WGN + wn2) * NF + 2 * (16 * j + v) + st) * 64 + 32 * h;
#pragma unroll
                    for (int l = 0; l < 32; l += 4) {
                        const f32x4 q4 = *(const f32x4 *)(row + l);
                        sum += (q4[0] + q4[1]) + (q4[2] + q4[3]);
                    }
                }
                return sum;
            };
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    float t1 = 0.f;
#pragma unroll
                    for (int i = 0; i < MI; ++i) t1 += acc[i][j][v];
                    scr[(wave * NF + 2 * (16 * j + v)) * 64 + ln] = t1;
                }
            barrier();
            for (int ch = tid; ch < BN; ch += NT) cmean[ch] = reduce(0, ch) / (float)nvalid;
            barrier();
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 m4 = *(const f32x4 *)(cmean + wn * 32 * NJ + 32 * j + 8 * g + 4 * ehi);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float t2 = 0.f;
#pragma unroll
                        for (int i = 0; i < MI; ++i) {
                            const float d = acc[i][j][4 * g + e] - m4[e];
                            t2 = wm * 32 * MI + 32 * i + el32 < nvalid ? fmaf(d, d, t2) : t2;
                        }
                        scr[(wave * NF + 2 * (16 * j + 4 * g + e) + 1) * 64 + ln] = t2;
                    }
                }
            barrier();
            {
                const int row = blockIdx.x * p.maxmc + mc;
                for (int ch = tid; ch < BN; ch += NT) {
                    p.partials[(size_t)row * 2 * p.K + n0 + ch] = cmean[ch];
                    p.partials[(size_t)row * 2 * p.K + p.K + n0 + ch] = reduce(1, ch);
                }
                if (n0 == 0 && tid == 0) counts[row] = (float)nvalid;
            }
            barrier();
        }
        float bj[NJ][16];
        if constexpr (EPI == EPI_BIAS_RELU || EPI == EPI_BIAS) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 b4 = p.bias ? *(const f32x4 *)(p.bias + n0 + wn * 32 * NJ + 32 * j + 8 * g + 4 * ehi)
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int e = 0; e < 4; ++e) bj[j][4 * g + e] = b4[e];
                }
        }
        // Staging: pixel px, channel chunk cc (8 channels) at px*STG_ROW + ((cc ^ (px & 15)) << 4).
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const int px = wm * 32 * MI + 32 * i + el32;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float a[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] = acc[i][j][4 * g + e];
                        if constexpr (EPI == EPI_BIAS_RELU) a[e] = fmaxf(a[e] + bj[j][4 * g + e], 0.f);
                        if constexpr (EPI == EPI_BIAS) a[e] += bj[j][4 * g + e];
                    }
                    const int cc = wn * 4 * NJ + 4 * j + g;
                    lds_write8(sbase + px * STG_ROW + ((cc ^ (px & 15)) << 4) + 8 * ehi,
                               u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])});
                    // one block at a time: keeps the accumulators from being copied out all at once
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        barrier();
        const __amdgpu_buffer_rsrc_t orr =
            __builtin_amdgcn_make_buffer_rsrc(p.out, 0, (int)((size_t)p.M * p.K * 2), 0x00020000);
        // 1 KB store instructions, SB per wave in flight: instruction s covers staging
        // bytes [1024 s, 1024 s + 1024) in pixel-major order.
        constexpr int NSI = BM * STG_ROW / 1024, SB = NW >= 8 ? 2 : 4;
        static_assert(NSI % (SB * NW) == 0, "store batches");
        for (int s0 = wave; s0 < NSI; s0 += SB * NW) {
            u32x4 v[SB];
            int off[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const int b = (s0 + NW * k) * 1024 + ln * 16;
                const int px = b / STG_ROW, cc = (b - px * STG_ROW) >> 4;
                v[k] = lds_read16u(sbase + px * STG_ROW + ((cc ^ (px & 15)) << 4));
                off[k] = px < nvalid ? 2 * ((cm0 + px) * p.K + n0) + 16 * cc : (int)0x80000000u;
            }
            lgkm_wait<0>();
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                after_wait(v[k]);
                __builtin_amdgcn_raw_buffer_store_b128(v[k], orr, off[k], 0, 0);
            }
        }
    };

    // ---- main loop over the slice sequence ----
    // (loads never run past the current chunk: its epilogue overwrites the slice buffers)
    const int npro = min(NSTAGE - 1, min(total, p.ksteps));
    for (int g = 0; g < npro; ++g) dma_issue(g);
    if (total > 0) {
        vm_wait_steps<LMIN>(npro - 1);
        barrier();
        read_frags(af[0], bf[0], 0, 0);
    }
    zero_acc();
    // One chunk's slices g0 .. g0 + ksteps - 1 with NB pixel blocks per wave; the MFMA
    // count is fixed for the whole chunk (the switch below picks the instance), so the
    // accumulators stay in place through the loop.
    auto chunk_loop = [&](auto nbc, int g0) __attribute__((always_inline)) {
        constexpr int NB = decltype(nbc)::value;
        const int lim = g0 + p.ksteps;   // the chunk's last slice bounds the loads
        for (int ks = 0; ks < p.ksteps; ++ks) {
            const int g = g0 + ks;
            // k-steps 0 .. KH-2: read the next k-step's fragments, then the MFMAs of this one;
            // the next slice's loads go out behind the first MFMAs, which run meanwhile
#pragma unroll
            for (int kh = 0; kh + 1 < KH; ++kh) {
                bf16x8 (&an)[NJ] = af[(kh + 1) & 1];
                bf16x8 (&bn)[MI] = bf[(kh + 1) & 1];
                read_frags(an, bn, g, kh + 1);
                lgkm_wait<MI + NJ>();
#pragma unroll
                for (int j = 0; j < NJ; ++j) after_wait(af[kh & 1][j]);
#pragma unroll
                for (int i = 0; i < MI; ++i) after_wait(bf[kh & 1][i]);
                __builtin_amdgcn_sched_barrier(0);
                mfma_set<MI, NJ, NB>(acc, af[kh & 1], bf[kh & 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (kh == 0 && g + NSTAGE - 1 < lim) dma_issue(g + NSTAGE - 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            // last k-step: its fragments in, the next slice landed, every wave past this
            // slice's buffer; then the next slice's first fragments under its MFMAs
            lgkm_wait<0>();
#pragma unroll
            for (int j = 0; j < NJ; ++j) after_wait(af[(KH - 1) & 1][j]);
#pragma unroll
            for (int i = 0; i < MI; ++i) after_wait(bf[(KH - 1) & 1][i]);
            if (g + 1 < lim) vm_wait_steps<LMIN>(min(NSTAGE - 2, lim - 2 - g));
            barrier();
            if (ks + 1 < p.ksteps) read_frags(af[0], bf[0], g + 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            mfma_set<MI, NJ, NB>(acc, af[(KH - 1) & 1], bf[(KH - 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int c = 0; c < nchunk; ++c) {
        const int g0 = c * p.ksteps;
        // MFMA instances by this wave's pixel blocks in the chunk, rounded up to MI, 4, 2, 1
        // or 0 (a partial block costs as much as a full one)
        const int mc = c / p.ntn;
        const int nv = min(BM, r1 - (r0 + mc * BM)) - wm * 32 * MI;
        const int nbv = nv <= 0 ? 0 : min(MI, (nv + 31) / 32);
        if (nbv > 4 || nbv == MI || (MI <= 4 && nbv > 2)) chunk_loop(std::integral_constant<int, MI>{}, g0);
        else if (nbv > 2) { if constexpr (MI > 4) chunk_loop(std::integral_constant<int, 4>{}, g0); }
        else if (nbv == 2) { if constexpr (MI > 2) chunk_loop(std::integral_constant<int, 2>{}, g0); }
        else if (nbv == 1) { if constexpr (MI > 1) chunk_loop(std::integral_constant<int, 1>{}, g0); }
        else chunk_loop(std::integral_constant<int, 0>{}, g0);
        epilogue(c);
        zero_acc();
        if (g0 + p.ksteps < total) {
            // the slice buffers held the staging tile: every wave is past its store reads
            // before the next chunk's first slices load
            barrier();
            const int np = min(NSTAGE - 1, p.ksteps);
            for (int g = 0; g < np; ++g) dma_issue(g0 + p.ksteps + g);
            vm_wait_steps<LMIN>(np - 1);
            barrier();
            read_frags(af[0], bf[0], g0 + p.ksteps, 0);
        }
    }

}

struct IgConfig {
    int mi, nj, wgm, wgn, bk, nstage;
    int bm() const { return 32 * mi * wgm; }
    int bn() const { return 32 * nj * wgn; }
    int nw() const { return wgm * wgn; }
};

int ig_grid(const ConvGeom &g) { return std::min(256, (g.M + 31) / 32); }
int ig_rows_per_wg(const ConvGeom &g) { return (g.M + ig_grid(g) - 1) / ig_grid(g); }

// PLAN_IG_224X256: chunks of 224 pixels x 256 channels, eight waves side by side over the
// channels (two per SIMD).  PLAN_IG_448X128: chunks of 448 pixels x 128 channels, eight
// waves in a 2 x 4 grid of 224 x 32 wave tiles.  Slices of 64 reduction elements (whole
// 128-byte rows) when C % 64 == 0, two in flight; else of 32, four in flight.  The
// epilogue stages in the slice buffers.
IgConfig ig_config(const ConvGeom &g, int plan)
{
    const bool wide = g.C % 64 == 0;
    if (plan == PLAN_IG_224X256) return IgConfig{7, 1, 1, 8, wide ? 64 : 32, wide ? 2 : 4};
    return IgConfig{7, 1, 2, 4, wide ? 64 : 32, wide ? 2 : 4};
}

size_t ig_lds_bytes(const ConvGeom &g, int epi, int plan)
{
    const IgConfig c = ig_config(g, plan);
    const size_t stage = (size_t)c.nstage * (c.bm() + c.bn()) * 2 * c.bk;
    const size_t scr = epi == EPI_STATS ? (size_t)c.nw() * 64 * c.nj * 32 * 4 : 0;
    const size_t stg = std::max((size_t)c.bm() * 2 * c.bn(), scr);
    const size_t stats = epi == EPI_STATS ? (size_t)c.bn() * 4 : 0;   // a chunk's channel means
    return std::max(stage, stg) + stats;
}

template <int MI, int NJ, int WGM, int WGN, int BK, int NSTAGE, int EPI>
hipError_t ig_launch_one(const IgParams &prm, int grid, size_t lds, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    const hipError_t e = raise_lds_limit((const void *)conv_igemm_kernel<MI, NJ, WGM, WGN, BK, NSTAGE, EPI>, (int)lds);
    if (e != hipSuccess) return e;
    return launch(conv_igemm_kernel<MI, NJ, WGM, WGN, BK, NSTAGE, EPI>, dim3(grid), dim3(64 * WGM * WGN),
                  (uint32_t)lds, st, e0, e1, prm);
}

template <int MI, int NJ, int WGM, int WGN, int BK, int NSTAGE>
hipError_t ig_launch_cfg(int epi, const IgParams &prm, int grid, size_t lds, hipStream_t st, hipEvent_t e0,
                         hipEvent_t e1)
{
    switch (epi) {
    case EPI_STATS: return ig_launch_one<MI, NJ, WGM, WGN, BK, NSTAGE, EPI_STATS>(prm, grid, lds, st, e0, e1);
    case EPI_BIAS_RELU:
        return ig_launch_one<MI, NJ, WGM, WGN, BK, NSTAGE, EPI_BIAS_RELU>(prm, grid, lds, st, e0, e1);
    case EPI_BIAS: return ig_launch_one<MI, NJ, WGM, WGN, BK, NSTAGE, EPI_BIAS>(prm, grid, lds, st, e0, e1);
    default: return ig_launch_one<MI, NJ, WGM, WGN, BK, NSTAGE, EPI_PLAIN>(prm, grid, lds, st, e0, e1);
    }
}

}  // namespace

bool igemm_eligible(const ConvGeom &g, int epi, int plan)
{
    if (plan != PLAN_IG_224X256 && plan != PLAN_IG_448X128) return false;
    if (g.C % 32 != 0 || g.M <= 0 || g.R > 16 || g.S > 16) return false;
    const IgConfig c = ig_config(g, plan);
    if (g.K % c.bn() != 0) return false;
    const double xbytes = 2.0 * g.N * g.H * g.W * g.C, obytes = 2.0 * g.M * g.K, wbytes = 2.0 * g.K * g.Kg;
    if (xbytes >= 2147483648.0 || obytes >= 2147483648.0 || wbytes >= 2147483648.0) return false;
    return ig_lds_bytes(g, epi, plan) <= 160 * 1024;
}

int ig_maxmc(const ConvGeom &g, int plan)
{
    return (ig_rows_per_wg(g) + ig_config(g, plan).bm() - 1) / ig_config(g, plan).bm();
}

int igemm_partial_rows(const ConvGeom &g, int plan) { return ig_grid(g) * ig_maxmc(g, plan); }

hipError_t launch_conv_igemm(const ConvGeom &g, int epi, int plan, const uint16_t *x, const uint16_t *w,
                             const float *bias, uint16_t *out, float *partials, hipStream_t st, hipEvent_t e0,
                             hipEvent_t e1)
{
    const IgConfig c = ig_config(g, plan);
    IgParams prm;
    prm.x = x;
    prm.w = w;
    prm.bias = bias;
    prm.out = out;
    prm.partials = partials;
    prm.N = g.N;
    prm.R = g.R;
    prm.H = g.H; prm.W = g.W; prm.C = g.C; prm.K = g.K; prm.S = g.S;
    prm.sh = g.sh; prm.sw = g.sw; prm.ph = g.ph; prm.pw = g.pw;
    prm.P = g.P; prm.Q = g.Q; prm.M = g.M; prm.Kg = g.Kg;
    prm.ksteps = g.Kg / c.bk;
    prm.rows_per_wg = ig_rows_per_wg(g);
    prm.ntn = g.K / c.bn();
    prm.maxmc = ig_maxmc(g, plan);
    const int grid = ig_grid(g);
    const size_t lds = ig_lds_bytes(g, epi, plan);
    if (c.wgm == 1) {
        if (c.bk == 64) return ig_launch_cfg<7, 1, 1, 8, 64, 2>(epi, prm, grid, lds, st, e0, e1);
        return ig_launch_cfg<7, 1, 1, 8, 32, 4>(epi, prm, grid, lds, st, e0, e1);
    }
    if (c.bk == 64) return ig_launch_cfg<7, 1, 2, 4, 64, 2>(epi, prm, grid, lds, st, e0, e1);
    return ig_launch_cfg<7, 1, 2, 4, 32, 4>(epi, prm, grid, lds, st, e0, e1);
}

}  // namespace cbr
