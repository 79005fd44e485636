// conv3x3_c64.hip -- persistent 3x3 / stride 1 / pad 1 convolution with 64 input and 64
// output channels (the CBR page's N=256, 56x56, 64-channel workload), fused with the
// per-channel sum and sum of squares of its output (the conv + genstats step of the CBR
// page's training forward, section 4.1).
//
// One 512-thread workgroup per compute unit walks whole images in steps of TP = 4
// output rows.  In LDS it keeps
//   - the whole filter, 64 x 576 bf16, rows padded to 1168 bytes;
//   - a ring of 10 input rows: the 6 rows a step reads (its output rows +-1) and the 4
//     rows of the next step, which stream in while the step computes.  Row h (-1 <= h
//     <= H) lives in slot (h + 1) % 10; the padding rows -1 and H are zero slots.  A slot
//     holds W + 2 pixels of 64 channels (zero columns at both ends), 128 bytes each, whose
//     eight 16-byte channel chunks are stored XOR-permuted by (pixel / 2) % 8, so that
//     16 consecutive pixels of one fragment read hit 16 distinct 4-bank groups.
// Input rows are copied from HBM straight into their slot with global-to-LDS loads (no
// register staging, no separate ring write): a wave's load instruction moves 8 pixels,
// and each lane fetches the channel chunk that the permutation puts in its 16 bytes.
// Each input row is read from HBM once and serves all nine taps.
//
// GEMM mapping: v_mfma_f32_32x32x16_bf16 with the filter as the A operand (32 output
// channels) and the input pixels as the B operand (32 pixels), so each lane ends up
// holding 4 consecutive output channels of one pixel (8-byte stores of z).  A step has
// TP*W/32 pixel blocks (7 for W = 56) x 2 channel blocks.  Wave w owns channel block
// w % 2 and a quarter of the pixel blocks; waves w and w ^ 4 share a SIMD and get
// quarters (1, 0) or (3, 2), so every SIMD holds about half of one channel block.
// A full step's z stores are issued during the next step's k-loop, so the z traffic
// streams under the MFMAs instead of leaving as one burst per step.
// The statistics are accumulated per lane in fp32 registers across the whole persistent
// loop and reduced across lanes and waves once at the end: one partial per workgroup.
#include <hip/hip_ext.h>

#include "cbr_launch.h"

namespace cbr {
namespace {

constexpr int HC = 64;                  // input channels
constexpr int HK = 64;                  // output channels
constexpr int TP = 4;                   // output rows per step
constexpr int NSLOT = 10;               // ring slots: TP + 2 read, TP incoming
constexpr int WROW = 9 * HC * 2 + 16;   // bytes per filter row (576 bf16 + 16 bytes of padding)
constexpr int WBYTES = HK * WROW;       // 74,752
constexpr int PXB = HC * 2;             // bytes per staged pixel
constexpr int NT = 512;                 // threads: 8 waves, two per SIMD
constexpr int MAXW = 56;

struct HaloParams {
    const uint16_t *x;
    const uint16_t *w;
    uint16_t *z;
    float *partials;       // [gridDim.x][2][64]
    int N, H, W;
    int slot_bytes;        // (W + 2) * PXB
    uint32_t invW;         // ceil(65536 / W): v / W == (v * invW) >> 16 for v * W <= 65536
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ int div_w(int v, uint32_t invW) { return (int)(((uint32_t)v * invW) >> 16); }

// Chunk permutation of staged pixel u: channel chunk c is stored at position c ^ perm(u).
__device__ __forceinline__ int perm(int u) { return (u >> 1) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// Per pixel block: LDS byte address of staged pixel q + sx in the slot of tap row r
// (xb[r][sx]), and the lane's chunk permutation of those pixels, pre-shifted and with
// the lane's k-half folded in (cx[sx] = (hi ^ perm(q + sx)) << 4): the fragment of
// 16-channel chunk kc is at xb[r][sx] + ((32 * kc) ^ cx[sx]).
struct BlockAddr {
    int xb[3][3];
    int cx[3];
};

// Bf16 results of the previous full step, waiting to be stored: block bb, channel
// group g at byte offset off[bb] + 16*g of buffer zr.
struct Pending {
    u32x2 data[2][4];
    int off[2];
    __amdgpu_buffer_rsrc_t zr;
};

// The 36 k-steps of one step (9 taps x 4 chunks of 16 channels) for the pixel blocks in
// MASK (bit bb: block b0 + bb).  A wave runs only one or two MFMAs per k-step, so its
// fragments are read KD - 1 k-steps ahead (KD register sets) to cover the LDS latency.
// With PM, the previous full step's results (blocks in PM) are stored in k-steps 2, 6,
// ..., 30, so that they stream under the MFMAs.
constexpr int KD = 2;

template <uint32_t MASK, uint32_t PM>
__device__ __forceinline__ void kloop(const uint8_t *lds, int wa, const BlockAddr (&ba)[2], f32x16 (&acc)[2],
                                      const Pending &pend)
{
    bf16x8 wf[KD], xf[KD][2];
    auto rd = [&](int t, int b) {
        const int tap = t >> 2, kc = t & 3, r = tap / 3, sx = tap - 3 * r;
        wf[b] = *(const bf16x8 *)(lds + wa + tap * 128 + kc * 32);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
            if (MASK & (1u << bb))
                xf[b][bb] = *(const bf16x8 *)(lds + ba[bb].xb[r][sx] + ((32 * kc) ^ ba[bb].cx[sx]));
    };
#pragma unroll
    for (int t = 0; t < KD - 1; ++t) rd(t, t);
#pragma unroll
    for (int t = 0; t < 36; ++t) {
        if (t + KD - 1 < 36) rd(t + KD - 1, (t + KD - 1) % KD);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
            if (MASK & (1u << bb))
                acc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t % KD], xf[t % KD][bb],
                                                                  t == 0 ? f32x16{} : acc[bb], 0, 0, 0);
        if constexpr (PM != 0) {
            const int sidx = (t - 2) / 4;   // store slot of k-steps 2, 6, ..., 30
            if (t >= 2 && (t - 2) % 4 == 0 && sidx < 8 && (PM & (1u << (sidx >> 2))))
                __builtin_amdgcn_raw_buffer_store_b64(pend.data[sidx >> 2][sidx & 3], pend.zr,
                                                      pend.off[sidx >> 2] + 16 * (sidx & 3), 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Full step: statistics of the blocks in MASK, and their results packed into pend.
// The lane holds, for pixel l32 of each block, channels 32j + 8g + 4hi + e in
// acc[bb][4g + e] (32x32x16 layout: row 8*(v/4) + 4*(l/32) + v%4).
template <uint32_t MASK>
__device__ __forceinline__ void finish(const f32x16 (&acc)[2], const int (&zoff)[2], __amdgpu_buffer_rsrc_t zr,
                                       float (&s1)[4][4], float (&s2)[4][4], Pending &pend)
{
    pend.zr = zr;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        if (!(MASK & (1u << bb))) continue;
        pend.off[bb] = zoff[bb];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float a0 = acc[bb][4 * g], a1 = acc[bb][4 * g + 1];
            const float a2 = acc[bb][4 * g + 2], a3 = acc[bb][4 * g + 3];
            pend.data[bb][g] = u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
            s1[g][0] += a0; s2[g][0] = fmaf(a0, a0, s2[g][0]);
            s1[g][1] += a1; s2[g][1] = fmaf(a1, a1, s2[g][1]);
            s1[g][2] += a2; s2[g][2] = fmaf(a2, a2, s2[g][2]);
            s1[g][3] += a3; s2[g][3] = fmaf(a3, a3, s2[g][3]);
        }
    }
}

template <uint32_t PM>
__device__ __forceinline__ void flush(const Pending &pend)
{
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
        if (PM & (1u << bb))
#pragma unroll
            for (int g = 0; g < 4; ++g)
                __builtin_amdgcn_raw_buffer_store_b64(pend.data[bb][g], pend.zr, pend.off[bb] + 16 * g, 0, 0);
}

// Steps with missing pixels: statistics and immediate stores of the lanes in use.
__device__ __forceinline__ void epilogue_masked(const f32x16 (&acc)[2], const int (&zoff)[2], const bool (&use)[2],
                                                __amdgpu_buffer_rsrc_t zr, float (&s1)[4][4], float (&s2)[4][4])
{
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        if (!use[bb]) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float a0 = acc[bb][4 * g], a1 = acc[bb][4 * g + 1];
            const float a2 = acc[bb][4 * g + 2], a3 = acc[bb][4 * g + 3];
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)}, zr,
                                                  zoff[bb] + 16 * g, 0, 0);
            s1[g][0] += a0; s2[g][0] = fmaf(a0, a0, s2[g][0]);
            s1[g][1] += a1; s2[g][1] = fmaf(a1, a1, s2[g][1]);
            s1[g][2] += a2; s2[g][2] = fmaf(a2, a2, s2[g][2]);
            s1[g][3] += a3; s2[g][3] = fmaf(a3, a3, s2[g][3]);
        }
    }
}

__global__ __launch_bounds__(NT, 1) void conv3x3_c64_stats_kernel(HaloParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t *wl = lds;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, W = p.W, SLOT = p.slot_bytes;
    const uint32_t invW = p.invW;
    const int spi = (H + TP - 1) / TP;                        // steps per image
    const int nimg = (p.N - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int hi = lane >> 5;                                 // k-half of the MFMA operands
    const int l32 = lane & 31;
    const int ipr = W / 8;                                    // 8-pixel load instructions per row
    // Wave w runs on SIMD w % 4 beside wave w ^ 4.  Channel block j = w & 1; the pixel
    // blocks are cut into quarters q0..q3 and SIMD pairs take (q1, q0) or (q3, q2).
    const int j = wave & 1;
    const int quarter = (wave < 4) ? ((wave & 2) ? 3 : 1) : ((wave & 2) ? 2 : 0);

    // Stages input rows h0 .. h0 + nrows - 1 (each -1 <= h <= H + 3) of image n into their
    // slots: image rows by global-to-LDS loads, the others as zeros.  Instruction gi
    // (row ri, pixels 8i .. 8i+7) is issued by wave gi % 8; lane l moves pixel 8i + l/8,
    // position l % 8, which holds channel chunk (l % 8) ^ perm(1 + 8i + l/8).
    auto stage_rows = [&](int n, int h0, int nrows) {
        for (int gi = wave; gi < nrows * ipr; gi += 8) {
            const int ri = gi / ipr, i = gi - ri * ipr;
            const int h = h0 + ri;
            const int dst = WBYTES + ((h + 1) % NSLOT) * SLOT + (1 + 8 * i) * PXB;   // wave-uniform
            if (h >= 0 && h < H) {
                const int u = 1 + 8 * i + (lane >> 3);
                const uint16_t *src =
                    p.x + ((size_t)(n * H + h) * W + 8 * i + (lane >> 3)) * HC + (((lane & 7) ^ perm(u)) * 8);
                __builtin_amdgcn_global_load_lds((const void *)src, (lds_u8 *)lds + dst, 16, 0, 0);
            } else {
                *(u32x4 *)(lds + dst + lane * 16) = u32x4{0, 0, 0, 0};
            }
        }
    };

    // Prologue: the filter into LDS (all of a thread's loads in flight first), the
    // padding columns of every slot zeroed, the first image's rows -1..4 staged.
    {
        constexpr int WCH = HK * 72 / NT;   // 9 filter chunks of 16 bytes per thread
        u32x4 wv[WCH];
#pragma unroll
        for (int i = 0; i < WCH; ++i) wv[i] = ((const u32x4 *)p.w)[tid + NT * i];
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const int c = tid + NT * i, row = c / 72, ch = c - row * 72;
            *(u32x4 *)(wl + row * WROW + ch * 16) = wv[i];
        }
    }
    for (int c = tid; c < NSLOT * 16; c += NT) {
        const int slot = c >> 4, col = (c & 8) ? W + 1 : 0;
        *(u32x4 *)(lds + WBYTES + slot * SLOT + col * PXB + (c & 7) * 16) = u32x4{0, 0, 0, 0};
    }
    if (nimg > 0) stage_rows(blockIdx.x, -1, TP + 2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Per-lane running statistics: channel 32*j + 8*g + 4*hi + e.
    float s1[4][4], s2[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s1[g][e] = 0.f;
            s2[g][e] = 0.f;
        }

    // Filter fragment base: row 32*j + l32, k-half hi (tap and chunk are immediates).
    const int wa = (32 * j + l32) * WROW + hi * 16;

    Pending pend;
    uint32_t pm = 0;   // blocks of the previous full step still to be stored
    for (int img = 0; img < nimg; ++img) {
        const int n = (int)blockIdx.x + img * (int)gridDim.x;
        if (img > 0) {
            // A new image: every wave is past the last step's reads; restage rows -1..4.
            stage_rows(n, -1, TP + 2);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        for (int s = 0; s < spi; ++s) {
            const int p0 = s * TP;
            const int rows_s = min(TP, H - p0);
            const int npix = rows_s * W;
            const int nblk = (npix + 31) >> 5;
            const int b0 = (quarter * nblk) >> 2, b1 = ((quarter + 1) * nblk) >> 2;   // blocks [b0, b1), <= 2
            const int nb = b1 - b0;
            const bool full = npix == nblk * 32;

            // The next step's rows p0 + 5 .. p0 + 8 stream into the 4 free slots.
            if (s + 1 < spi) stage_rows(n, p0 + TP + 1, TP);
            __builtin_amdgcn_sched_barrier(0);

            const __amdgpu_buffer_rsrc_t zr = make_rsrc(p.z + ((size_t)n * H + p0) * W * HK, npix * HK * 2);
            BlockAddr ba[2];
            int zoff[2];
            bool use[2];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int pi = 32 * (b0 + bb) + l32;
                const bool valid = pi < npix;
                const int pr = valid ? div_w(pi, invW) : 0;
                const int q = valid ? pi - pr * W : 0;
                use[bb] = valid && bb < nb;
                zoff[bb] = 2 * (pi * HK + 32 * j + 4 * hi);
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    int sl = (p0 % NSLOT) + pr + r;        // slot of input row p0 + pr + r - 1
                    if (sl >= NSLOT) sl -= NSLOT;
                    if (sl >= NSLOT) sl -= NSLOT;
#pragma unroll
                    for (int sx = 0; sx < 3; ++sx) ba[bb].xb[r][sx] = WBYTES + sl * SLOT + (q + sx) * PXB;
                }
#pragma unroll
                for (int sx = 0; sx < 3; ++sx) ba[bb].cx[sx] = (hi ^ perm(q + sx)) << 4;
            }

            f32x16 acc[2];
            if (full && nb == 2) {
                if (pm == 3u)
                    kloop<3u, 3u>(lds, wa, ba, acc, pend);
                else if (pm == 1u)
                    kloop<3u, 1u>(lds, wa, ba, acc, pend);
                else
                    kloop<3u, 0u>(lds, wa, ba, acc, pend);
                finish<3u>(acc, zoff, zr, s1, s2, pend);
                pm = 3u;
            } else if (full && nb == 1) {
                if (pm == 3u)
                    kloop<1u, 3u>(lds, wa, ba, acc, pend);
                else if (pm == 1u)
                    kloop<1u, 1u>(lds, wa, ba, acc, pend);
                else
                    kloop<1u, 0u>(lds, wa, ba, acc, pend);
                finish<1u>(acc, zoff, zr, s1, s2, pend);
                pm = 1u;
            } else {
                if (pm == 3u) flush<3u>(pend);
                if (pm == 1u) flush<1u>(pend);
                pm = 0;
                if (nb > 0) {
                    kloop<3u, 0u>(lds, wa, ba, acc, pend);
                    epilogue_masked(acc, zoff, use, zr, s1, s2);
                }
            }

            // The staged rows must have landed before any wave reads them: wait for this
            // wave's loads, then the barrier publishes every wave's.  The barrier also
            // frees the slots this step read for the step after next.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }
    if (pm == 3u) flush<3u>(pend);
    if (pm == 1u) flush<1u>(pend);

    // Cross-lane sum through LDS, in the filter area (no longer read: the last step's
    // barrier has passed; 64 KB <= WBYTES).  st[f][tid] holds entry f of the lane's
    // flattened [s1 | s2]: entry 16*which + 4*g + e is channel 32j + 8g + 4hi + e.
    float *st = (float *)wl;             // [32][NT]
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            st[(4 * g + e) * NT + tid] = s1[g][e];
            st[(16 + 4 * g + e) * NT + tid] = s2[g][e];
        }
    __syncthreads();
    // Thread (f, jj, h) sums the 128 lanes of channel block jj with hi == h: waves
    // jj, jj + 2, jj + 4, jj + 6 x 32 lanes, fixed order.
    if (tid < 128) {
        const int f = tid >> 2, jj = (tid >> 1) & 1, h = tid & 1;
        const f32x4 *row = (const f32x4 *)(st + f * NT + 32 * h);
        float a = 0.f;
#pragma unroll
        for (int w = jj; w < 8; w += 2)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4 q = row[16 * w + i];
                a += (q[0] + q[1]) + (q[2] + q[3]);
            }
        const int which = f >> 4, ge = f & 15;
        const int k = 32 * jj + 8 * (ge >> 2) + 4 * h + (ge & 3);
        p.partials[(size_t)blockIdx.x * 2 * HK + which * HK + k] = a;
    }
}

}  // namespace

bool halo_eligible(const ConvGeom &g)
{
    return g.C == HC && g.K == HK && g.R == 3 && g.S == 3 && g.sh == 1 && g.sw == 1 && g.ph == 1 &&
           g.pw == 1 && g.W >= 8 && g.W <= MAXW && g.W % 8 == 0 && g.P == g.H && g.Q == g.W;
}

int halo_grid(const ConvGeom &g) { return std::min(g.N, HALO_MAX_GRID); }

size_t halo_lds_bytes(const ConvGeom &g) { return WBYTES + (size_t)NSLOT * (g.W + 2) * PXB; }

hipError_t launch_conv3x3_c64_stats(const ConvGeom &g, const uint16_t *x, const uint16_t *w, uint16_t *z,
                                    float *partials, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    HaloParams prm{x, w, z, partials, g.N, g.H, g.W, (g.W + 2) * PXB, (65536u + g.W - 1) / g.W};
    const size_t lds = halo_lds_bytes(g);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)conv3x3_c64_stats_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)HALO_MAX_LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const dim3 grid(halo_grid(g)), block(NT);
    if (e0 || e1)
        hipExtLaunchKernelGGL(conv3x3_c64_stats_kernel, grid, block, (uint32_t)lds, st, e0, e1, 0, prm);
    else
        conv3x3_c64_stats_kernel<<<grid, block, lds, st>>>(prm);
    return hipGetLastError();
}

}  // namespace cbr
