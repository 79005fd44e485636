// conv3x3_c64.hip -- persistent 3x3 / stride 1 / pad 1 convolution with 64 input and 64
// output channels (the CBR page's N=256, 56x56, 64-channel workload), fused with the
// per-channel sum and sum of squares of its output (the conv + genstats step of the CBR
// page's training forward, section 4.1).
//
// One 256-thread workgroup per compute unit walks whole images in steps of TP = 8 output
// rows.  In LDS it keeps
//   - the whole filter, 64 x 576 bf16, rows padded to 1168 bytes;
//   - a ring of TP + 2 input rows (row h in slot (h + 10) % 10, so the padding rows -1
//     and H get slots too; those slots are zeroed while the window holds them).  Each
//     slot holds W + 2 pixels (zero padding columns at both ends) of 64 channels, pixels
//     padded to 144 bytes.
// The paddings make every 8 consecutive lanes of an MFMA fragment read hit 8 distinct
// 4-bank groups, and keep each fragment address a per-lane base plus a compile-time
// offset (tap and channel chunk).  Input rows come from HBM once and serve all nine
// taps.  While a step computes, the input rows of the next step are already in flight
// into registers.
//
// GEMM mapping: v_mfma_f32_32x32x16_bf16 with the filter as the A operand (32 output
// channels) and the input pixels as the B operand (32 pixels), so each lane ends up
// holding 4 consecutive output channels of one pixel (8-byte stores of z).  A step has
// (TP*W/32) pixel blocks x 2 channel blocks = 28 units for W = 56; each of the four
// waves owns a contiguous quarter of them (7 units, at most 4 pixel blocks).
// The statistics are accumulated per lane in fp32 registers across the whole persistent
// loop and reduced across lanes and waves once at the end: one partial per workgroup.
#include <hip/hip_ext.h>

#include "cbr_launch.h"

namespace cbr {
namespace {

constexpr int HC = 64;                  // input channels
constexpr int HK = 64;                  // output channels
constexpr int TP = 8;                   // output rows per step
constexpr int NSLOT = TP + 2;           // input-row ring slots
constexpr int WROW = 9 * HC * 2 + 16;   // bytes per filter row (576 bf16 + 16 bytes of padding)
constexpr int WBYTES = HK * WROW;       // 74,752
constexpr int PXB = HC * 2 + 16;        // bytes per staged pixel (64 bf16 + 16 bytes of padding)
constexpr int NT = 256;
constexpr int PF = 16;                  // 16-byte prefetch chunks per thread

struct HaloParams {
    const uint16_t *x;
    const uint16_t *w;
    uint16_t *z;
    float *partials;       // [gridDim.x][2][64]
    int N, H, W;
    int slot_bytes;        // (W + 2) * PXB
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int ring_slot(int h) { return (h + NSLOT) % NSLOT; }   // h >= -1

// Fragment reads of k-step t (tap t/4 = (r, sx), 16-channel chunk t%4) into wf/xf:
// per-lane bases plus compile-time offsets.
__device__ __forceinline__ void load_frags(int t, const uint8_t *wl, const uint8_t *ring, const int (&wa)[2],
                                          const int (&xa)[4][3], bf16x8 (&wf)[2], bf16x8 (&xf)[4])
{
    const int tap = t >> 2, kc = t & 3, r = tap / 3, sx = tap - 3 * r;
#pragma unroll
    for (int j = 0; j < 2; ++j) wf[j] = *(const bf16x8 *)(wl + wa[j] + tap * 128 + kc * 32);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) xf[bb] = *(const bf16x8 *)(ring + xa[bb][r] + sx * PXB + kc * 32);   // ring == LDS base
}

// Bit index (2*bb + j) of the u-th set bit of MASK: the u-th unit of a wave.
template <uint32_t MASK>
constexpr int unit_bit(int u)
{
    int c = 0;
    for (int b = 0; b < 8; ++b)
        if (MASK & (1u << b)) {
            if (c == u) return b;
            ++c;
        }
    return -1;
}

// Bf16 results of one full step, waiting to be stored: 7 units x 4 groups of 4 channels.
struct Pending {
    u32x2 data[7][4];
    uint16_t *dst[7];    // z address of channel 32j + 4hi of the lane's pixel, per unit
};

// The 36 k-steps of one step (9 taps x 4 chunks of 16 channels).  Fragments of k-step
// t+1 are read while the MFMAs of k-step t run.  MASK selects at compile time the
// (pixel block, channel block) slots that run (bit 2*bb + j).  When `stores` is set,
// the previous step's results (pend) are written out one 8-byte store per k-step, so
// that the z traffic streams during the MFMAs instead of arriving as one burst.
template <uint32_t MASK>
__device__ __forceinline__ void kloop(const uint8_t *wl, const uint8_t *ring, const int (&wa)[2],
                                      const int (&xa)[4][3], f32x16 (&acc)[4][2], bool stores,
                                      const Pending &pend)
{
    bf16x8 wf[2][2], xf[2][4];
    load_frags(0, wl, ring, wa, xa, wf[0], xf[0]);
#pragma unroll
    for (int t = 0; t < 36; ++t) {
        if (t + 1 < 36) load_frags(t + 1, wl, ring, wa, xa, wf[(t + 1) & 1], xf[(t + 1) & 1]);
        // Keep the reads of k-step t+1 ahead of the MFMAs of k-step t: the scheduler would
        // otherwise sink each read down to its use and expose the LDS latency.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (MASK & (1u << (2 * bb + j)))
                    acc[bb][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t & 1][j], xf[t & 1][bb], acc[bb][j],
                                                                         0, 0, 0);
        if constexpr (MASK != 0xFFu) {
            if (t < 28 && stores) *(u32x2 *)(pend.dst[t >> 2] + 8 * (t & 3)) = pend.data[t >> 2][t & 3];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Full step (every pixel valid): fold the unit results into the statistics and pack them
// into pend for the next k-loop to store.
template <uint32_t MASK>
__device__ __forceinline__ void finish_full(const f32x16 (&acc)[4][2], uint16_t *zrow, const int (&pix)[4], int hi,
                                            float (&s1)[2][4][4], float (&s2)[2][4][4], Pending &pend)
{
#pragma unroll
    for (int u = 0; u < 7; ++u) {
        const int bit = unit_bit<MASK>(u), bb = bit >> 1, j = bit & 1;
        pend.dst[u] = zrow + (size_t)pix[bb] * HK + 32 * j + 4 * hi;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float a0 = acc[bb][j][4 * g], a1 = acc[bb][j][4 * g + 1];
            const float a2 = acc[bb][j][4 * g + 2], a3 = acc[bb][j][4 * g + 3];
            pend.data[u][g] = u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
            s1[j][g][0] += a0; s2[j][g][0] = fmaf(a0, a0, s2[j][g][0]);
            s1[j][g][1] += a1; s2[j][g][1] = fmaf(a1, a1, s2[j][g][1]);
            s1[j][g][2] += a2; s2[j][g][2] = fmaf(a2, a2, s2[j][g][2]);
            s1[j][g][3] += a3; s2[j][g][3] = fmaf(a3, a3, s2[j][g][3]);
        }
    }
}

__device__ __forceinline__ void flush(const Pending &pend)
{
#pragma unroll
    for (int u = 0; u < 7; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g) *(u32x2 *)(pend.dst[u] + 8 * g) = pend.data[u][g];
}

__global__ __launch_bounds__(NT, 1) void conv3x3_c64_stats_kernel(HaloParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t *wl = lds;
    uint8_t *ring = lds + WBYTES;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, W = p.W, SLOT = p.slot_bytes;
    const int spi = (H + TP - 1) / TP;                        // steps per image
    const int nimg = (p.N - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int nsteps = nimg * spi;
    const int hi = lane >> 5;                                 // k-half of the MFMA operands
    const int l32 = lane & 31;

    // Filter -> LDS (72 chunks of 16 bytes per row).
    for (int c = tid; c < HK * 72; c += NT) {
        const int row = c / 72, ch = c - row * 72;
        *(u32x4 *)(wl + row * WROW + ch * 16) = ((const u32x4 *)p.w)[c];
    }
    // Zero the padding columns of every ring slot (row loads never write them).
    for (int c = tid; c < NSLOT * 16; c += NT) {
        const int slot = c >> 4, col = (c & 8) ? W + 1 : 0;
        *(u32x4 *)(ring + slot * SLOT + col * PXB + (c & 7) * 16) = u32x4{0, 0, 0, 0};
    }

    // Rows loaded for step t: s == 0 -> rows 0..min(H-1, TP); else s*TP+1..min(H-1, s*TP+TP).
    auto step_img = [&](int t, int &n, int &s) {
        n = (int)blockIdx.x + (t / spi) * (int)gridDim.x;
        s = t - (t / spi) * spi;
    };
    u32x4 pf[PF];
    auto load_rows = [&](int t) {
        int n, s;
        step_img(t, n, s);
        const int lo = s == 0 ? 0 : s * TP + 1;
        const int hiw = min(H - 1, s * TP + TP);
        const int total = (hiw - lo + 1) * W * 8;
        const u32x4 *src = (const u32x4 *)(p.x + ((size_t)n * H + lo) * W * HC);
#pragma unroll
        for (int i = 0; i < PF; ++i) pf[i] = src[min(tid + NT * i, total - 1)];   // extra lanes re-read a valid chunk
    };
    // Writes the rows of step t into the ring and zeroes the slots of the padding rows
    // -1 (first step of an image) and H (last step) that the step's window holds.
    auto store_rows = [&](int t) {
        int n, s;
        step_img(t, n, s);
        const int lo = s == 0 ? 0 : s * TP + 1;
        const int hiw = min(H - 1, s * TP + TP);
        const int total = (hiw - lo + 1) * W * 8;
        // chunk c = tid + 256*i: channel chunk tid % 8, pixel (tid / 8 + 32*i) of the rows
        // block, walked incrementally (row rr, column px).
        int px = tid >> 3, rr = 0;
        while (px >= W) { px -= W; ++rr; }
        int slot = ring_slot(lo + rr);
        const int choff = (tid & 7) * 16 + PXB;          // + one padding column
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            if (tid + NT * i < total) *(u32x4 *)(ring + slot * SLOT + px * PXB + choff) = pf[i];
            px += NT / 8;
            while (px >= W) {
                px -= W;
                slot = slot + 1 == NSLOT ? 0 : slot + 1;
            }
        }
        const bool top = s == 0, bottom = s == spi - 1;
        for (int c = tid; c < W * 8; c += NT) {
            const int off = (c / 8 + 1) * PXB + (c & 7) * 16;
            if (top) *(u32x4 *)(ring + ring_slot(-1) * SLOT + off) = u32x4{0, 0, 0, 0};
            if (bottom) *(u32x4 *)(ring + ring_slot(H) * SLOT + off) = u32x4{0, 0, 0, 0};
        }
    };

    // Per-lane running statistics: channel 32*j + 8*g + 4*hi + e.
    float s1[2][4][4], s2[2][4][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s1[j][g][e] = 0.f;
                s2[j][g][e] = 0.f;
            }

    // Filter fragment base: row 32*j + l32, k-half hi (tap and chunk are immediates).
    int wa[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) wa[j] = (32 * j + l32) * WROW + hi * 16;

    // Step order: prefetch the rows of t+1 (the register buffer was emptied into the ring
    // by the previous step); k-loop(t), which also stores the previous full step's z;
    // statistics + packing of step t; barrier; rows of t+1 into the ring; barrier.
    if (nsteps > 0) load_rows(0);
    __syncthreads();
    if (nsteps > 0) store_rows(0);
    __syncthreads();

    Pending pend;
    bool have_pend = false;
    for (int t = 0; t < nsteps; ++t) {
        int n, s;
        step_img(t, n, s);
        const int p0 = s * TP;
        const int rows_s = min(TP, H - p0);
        const int npix = rows_s * W;
        const int nblk = (npix + 31) >> 5;
        const int U = 2 * nblk;
        const int u0 = (wave * U) >> 2, u1 = ((wave + 1) * U) >> 2;
        const int b0 = u0 >> 1;
        uint32_t act = 0;   // bit (2*bb + j): unit (b0 + bb, j) belongs to this wave
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int u = 2 * (b0 + bb) + j;
                if (u >= u0 && u < u1) act |= 1u << (2 * bb + j);
            }
        act = __builtin_amdgcn_readfirstlane(act);
        const bool full = npix == nblk * 32;

        if (t + 1 < nsteps) load_rows(t + 1);

        // Fragment base of each pixel block and tap row: slot of input row p + r - 1,
        // column q (tap column sx adds sx pixels), k-half hi.  Lanes past the last pixel
        // read any in-range data; their results are dropped.
        int xa[4][3], pix[4];
        bool valid[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int pi = 32 * (b0 + bb) + l32;
            valid[bb] = pi < npix;
            const int pr = valid[bb] ? pi / W : 0;
            const int q = valid[bb] ? pi - pr * W : 0;
            pix[bb] = pi;
#pragma unroll
            for (int r = 0; r < 3; ++r) xa[bb][r] = WBYTES + ring_slot(p0 + pr + r - 1) * SLOT + q * PXB + hi * 16;
        }

        f32x16 acc[4][2];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[bb][j][v] = 0.f;

        uint16_t *zrow = p.z + ((size_t)n * H + p0) * W * HK;
        // Full steps give every wave 7 units in one of two patterns (skip the last or the
        // first unit of its 4 x 2 slots); those run branch-free and defer their stores to
        // the next k-loop.  Other (partial) steps run all 8 slots and store at once.
        if (full && act == 0x7Fu) {
            kloop<0x7Fu>(lds, lds, wa, xa, acc, have_pend, pend);
            finish_full<0x7Fu>(acc, zrow, pix, hi, s1, s2, pend);
            have_pend = true;
        } else if (full && act == 0xFEu) {
            kloop<0xFEu>(lds, lds, wa, xa, acc, have_pend, pend);
            finish_full<0xFEu>(acc, zrow, pix, hi, s1, s2, pend);
            have_pend = true;
        } else {
            if (have_pend) flush(pend);
            have_pend = false;
            kloop<0xFFu>(lds, lds, wa, xa, acc, false, pend);
            // Epilogue: lane holds, for pixel l32 of each block, channels 32j + 8g + 4hi + e
            // in acc[bb][j][4g + e] (32x32x16 layout: row 8*(v/4) + 4*(l/32) + v%4).
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (!(act & (1u << (2 * bb + j))) || !valid[bb]) continue;
                    uint16_t *zp = zrow + (size_t)pix[bb] * HK + 32 * j + 4 * hi;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float a0 = acc[bb][j][4 * g], a1 = acc[bb][j][4 * g + 1];
                        const float a2 = acc[bb][j][4 * g + 2], a3 = acc[bb][j][4 * g + 3];
                        *(u32x2 *)(zp + 8 * g) = u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
                        s1[j][g][0] += a0; s2[j][g][0] = fmaf(a0, a0, s2[j][g][0]);
                        s1[j][g][1] += a1; s2[j][g][1] = fmaf(a1, a1, s2[j][g][1]);
                        s1[j][g][2] += a2; s2[j][g][2] = fmaf(a2, a2, s2[j][g][2]);
                        s1[j][g][3] += a3; s2[j][g][3] = fmaf(a3, a3, s2[j][g][3]);
                    }
                }
        }

        __syncthreads();                 // every wave is done reading the ring for step t
        if (t + 1 < nsteps) store_rows(t + 1);
        __syncthreads();
    }
    if (have_pend) flush(pend);

    // The ring is no longer read (the last step's barriers have passed).
    // Lanes sharing hi hold the same channel set: reduce over the 32 lanes of each half.
    float *red = (float *)ring;          // [4 waves][2][64]
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float a = s1[j][g][e], b = s2[j][g][e];
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) {
                    a += __shfl_xor(a, o);
                    b += __shfl_xor(b, o);
                }
                if (l32 == 0) {
                    const int k = 32 * j + 8 * g + 4 * hi + e;
                    red[(wave * 2 + 0) * HK + k] = a;
                    red[(wave * 2 + 1) * HK + k] = b;
                }
            }
    __syncthreads();
    if (tid < 2 * HK) {
        const int which = tid / HK, k = tid - which * HK;
        float a = 0.f;
        for (int w = 0; w < 4; ++w) a += red[(w * 2 + which) * HK + k];
        p.partials[(size_t)blockIdx.x * 2 * HK + which * HK + k] = a;
    }
}

}  // namespace

bool halo_eligible(const ConvGeom &g)
{
    return g.C == HC && g.K == HK && g.R == 3 && g.S == 3 && g.sh == 1 && g.sw == 1 && g.ph == 1 &&
           g.pw == 1 && g.W >= 2 && (TP + 1) * g.W * 8 <= PF * NT && g.P == g.H && g.Q == g.W;
}

int halo_grid(const ConvGeom &g) { return std::min(g.N, HALO_MAX_GRID); }

size_t halo_lds_bytes(const ConvGeom &g) { return WBYTES + (size_t)NSLOT * (g.W + 2) * PXB; }

hipError_t launch_conv3x3_c64_stats(const ConvGeom &g, const uint16_t *x, const uint16_t *w, uint16_t *z,
                                    float *partials, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    HaloParams prm{x, w, z, partials, g.N, g.H, g.W, (g.W + 2) * PXB};
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
