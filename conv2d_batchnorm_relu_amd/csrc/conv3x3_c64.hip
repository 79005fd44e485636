// conv3x3_c64.hip -- persistent 3x3 / stride 1 / pad 1 convolution with 64 input and 64
// output channels (the CBR page's N=256, 56x56, 64-channel workload), fused with the
// per-channel sum and sum of squares of its output (the conv + genstats step of the CBR
// page's training forward, section 4.1).
//
// One 512-thread workgroup per compute unit walks whole images in steps of TP = 8 output
// rows.  In LDS it keeps
//   - the whole filter, 64 x 576 bf16, rows padded to 1168 bytes;
//   - a ring of TP + 2 input rows (row h in slot (h + 10) % 10, so the padding rows -1
//     and H get slots too; those slots are zeroed while the window holds them).  Each
//     slot holds W + 2 pixels (zero padding columns at both ends) of 64 channels, pixels
//     padded to 144 bytes.
// The paddings make every 16 consecutive lanes of an MFMA fragment read hit 16 distinct
// 4-bank groups, and keep each fragment address a per-lane base plus a compile-time
// offset (tap and channel chunk).  Input rows come from HBM once and serve all nine
// taps.  While a step computes, the input rows of the next step are already in flight
// into registers.
//
// GEMM mapping: v_mfma_f32_32x32x16_bf16 with the filter as the A operand (32 output
// channels) and the input pixels as the B operand (32 pixels), so each lane ends up
// holding 4 consecutive output channels of one pixel (8-byte stores of z).  A step has
// nblk = TP*W/32 pixel blocks (14 for W = 56) x 2 channel blocks.  Each of the eight
// waves owns one channel block j and a contiguous range of pixel blocks (a quarter of
// them), so one filter fragment and at most four pixel fragments feed its at most four
// MFMAs per k-step.  Two waves run on every SIMD, paired so that each SIMD gets half
// the pixel blocks of one channel block's ranges: while one wave stalls on memory,
// statistics or stores, the other keeps the matrix core busy.
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
constexpr int NT = 512;                 // threads: 8 waves, two per SIMD
constexpr int PF = 8;                   // 16-byte prefetch chunks per thread

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

__device__ __forceinline__ int div_w(int v, uint32_t invW) { return (int)(((uint32_t)v * invW) >> 16); }

// Buffer resource over [base, base + bytes): loads past the end return zeros, stores
// past the end are dropped (raw buffer, stride 0, 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// Fragment reads of k-step t (tap t/4 = (r, sx), 16-channel chunk t%4): the filter
// fragment of the wave's channel block and the pixel fragments of the blocks in MASK.
template <uint32_t MASK>
__device__ __forceinline__ void load_frags(int t, const uint8_t *lds, int wa, const int (&xa)[4][3], bf16x8 &wf,
                                          bf16x8 (&xf)[4])
{
    const int tap = t >> 2, kc = t & 3, r = tap / 3, sx = tap - 3 * r;
    wf = *(const bf16x8 *)(lds + wa + tap * 128 + kc * 32);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
        if (MASK & (1u << bb)) xf[bb] = *(const bf16x8 *)(lds + xa[bb][r] + sx * PXB + kc * 32);
}

// The 36 k-steps of one step (9 taps x 4 chunks of 16 channels) for the pixel blocks in
// MASK.  Fragments of k-step t+1 are read while the MFMAs of k-step t run.  The next
// step's input-row chunks are loaded in the first even k-steps, so that they stream
// under the MFMAs (lanes past the end of the rows block load zeros, never stored).
template <uint32_t MASK>
__device__ __forceinline__ void kloop(const uint8_t *lds, int wa, const int (&xa)[4][3], f32x16 (&acc)[4],
                                      __amdgpu_buffer_rsrc_t xr, int tid, u32x4 (&pf)[PF])
{
    bf16x8 wf[2], xf[2][4];
    load_frags<MASK>(0, lds, wa, xa, wf[0], xf[0]);
#pragma unroll
    for (int t = 0; t < 36; ++t) {
        if (t + 1 < 36) load_frags<MASK>(t + 1, lds, wa, xa, wf[(t + 1) & 1], xf[(t + 1) & 1]);
        // Keep the reads of k-step t+1 ahead of the MFMAs of k-step t: the scheduler would
        // otherwise sink each read down to its use and expose the LDS latency.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
            if (MASK & (1u << bb))
                acc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t & 1], xf[t & 1][bb],
                                                                  t == 0 ? f32x16{} : acc[bb], 0, 0, 0);
        if ((t & 1) == 0 && t / 2 < PF)
            pf[t / 2] = __builtin_amdgcn_raw_buffer_load_b128(xr, 16 * (tid + NT * (t / 2)), 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Statistics + bf16 stores of the pixel blocks in MASK: the lane holds, for pixel l32
// of each block, channels 32j + 8g + 4hi + e in acc[bb][4g + e] (32x32x16 layout: row
// 8*(v/4) + 4*(l/32) + v%4).  Blocks whose lane is past the last pixel (use false) are
// dropped.
template <uint32_t MASK>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[4], const int (&zoff)[4], const bool (&use)[4],
                                         __amdgpu_buffer_rsrc_t zr, float (&s1)[4][4], float (&s2)[4][4])
{
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
        if (!(MASK & (1u << bb)) || !use[bb]) continue;
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
    uint8_t *ring = lds + WBYTES;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, W = p.W, SLOT = p.slot_bytes;
    const uint32_t invW = p.invW;
    const int spi = (H + TP - 1) / TP;                        // steps per image
    const int nimg = (p.N - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int nsteps = nimg * spi;
    const int hi = lane >> 5;                                 // k-half of the MFMA operands
    const int l32 = lane & 31;
    // Wave w runs on SIMD w % 4 beside wave w ^ 4.  Channel block j = w & 1; the pixel
    // blocks are cut into quarters q0..q3 and SIMD pairs take (q1, q0) or (q3, q2), so
    // the two waves of a SIMD hold about half of one channel block's pixel blocks.
    const int j = wave & 1;
    const int quarter = (wave < 4) ? ((wave & 2) ? 3 : 1) : ((wave & 2) ? 2 : 0);

    // Input rows of step s of an image: s == 0 -> rows 0..min(H-1, TP); else
    // s*TP+1..min(H-1, s*TP+TP) (the rows above are already in the ring).
    auto rows_lo = [&](int s) { return s == 0 ? 0 : s * TP + 1; };
    auto rows_chunks = [&](int s) { return (min(H - 1, s * TP + TP) - rows_lo(s) + 1) * W * 8; };
    // Buffer over the rows block of step s of image n (loads past it return zeros).
    auto rows_rsrc = [&](int n, int s) {
        return make_rsrc(p.x + ((size_t)n * H + rows_lo(s)) * W * HC, rows_chunks(s) * 16);
    };
    // Writes the rows of step s (held in pf) into the ring, and zeroes the slots of the
    // padding rows -1 (first step of an image) and H (last step) that its window holds.
    // Chunk c = tid + NT*i of the block: pixel c/8 (row rr, column pc - rr*W), channel
    // chunk c%8.
    auto store_rows = [&](int s, const u32x4 (&pf)[PF]) {
        // An opaque copy of tid keeps the per-chunk address arithmetic here instead of
        // being hoisted out of the step loop (where its loop-invariant values would stay
        // live across every k-loop).
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int total = rows_chunks(s);
        const int slot_lo = rows_lo(s) % NSLOT;
        const int choff = (tid & 7) * 16 + PXB;          // + one padding column
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int c = tid + NT * i;
            if (c < total) {
                const int pc = c >> 3;
                const int rr = div_w(pc, invW);
                int slot = slot_lo + rr;
                if (slot >= NSLOT) slot -= NSLOT;
                *(u32x4 *)(ring + slot * SLOT + (pc - rr * W) * PXB + choff) = pf[i];
            }
        }
        const bool top = s == 0, bottom = s == spi - 1;
        for (int c = tid; c < W * 8; c += NT) {
            const int off = (c / 8 + 1) * PXB + (c & 7) * 16;
            if (top) *(u32x4 *)(ring + (NSLOT - 1) * SLOT + off) = u32x4{0, 0, 0, 0};
            if (bottom) *(u32x4 *)(ring + (H % NSLOT) * SLOT + off) = u32x4{0, 0, 0, 0};
        }
    };

    // Prologue: the first step's input rows and the whole filter in flight together,
    // then both into LDS.
    u32x4 pf[PF];
    if (nsteps > 0) {
        const __amdgpu_buffer_rsrc_t xr = rows_rsrc(blockIdx.x, 0);
#pragma unroll
        for (int i = 0; i < PF; ++i) pf[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, 16 * (tid + NT * i), 0, 0);
    }
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
    // Zero the padding columns of every ring slot (row stores never write them).
    for (int c = tid; c < NSLOT * 16; c += NT) {
        const int slot = c >> 4, col = (c & 8) ? W + 1 : 0;
        *(u32x4 *)(ring + slot * SLOT + col * PXB + (c & 7) * 16) = u32x4{0, 0, 0, 0};
    }
    if (nsteps > 0) store_rows(0, pf);
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

    // Step order: k-loop(t), which also loads the rows of t+1; statistics and z stores
    // of t; barrier; rows of t+1 into the ring; barrier.
    int n = blockIdx.x, s = 0;
    for (int t = 0; t < nsteps; ++t) {
        const int p0 = s * TP;
        const int rows_s = min(TP, H - p0);
        const int npix = rows_s * W;
        const int nblk = (npix + 31) >> 5;
        const int b0 = (quarter * nblk) >> 2, b1 = ((quarter + 1) * nblk) >> 2;   // blocks [b0, b1), <= 4
        const bool full = npix == nblk * 32;

        int sn = s + 1, nn = n;
        if (sn == spi) {
            sn = 0;
            nn += gridDim.x;
        }
        const bool next = t + 1 < nsteps;
        // Without a next step the k-loop re-reads this step's rows (always in bounds).
        const __amdgpu_buffer_rsrc_t xr = next ? rows_rsrc(nn, sn) : rows_rsrc(n, s);
        const __amdgpu_buffer_rsrc_t zr = make_rsrc(p.z + ((size_t)n * H + p0) * W * HK, npix * HK * 2);

        // Fragment base of each pixel block and tap row: slot of input row p + r - 1,
        // column q (tap column sx adds sx pixels), k-half hi.  Lanes past the last pixel
        // read any in-range data; their results are dropped.
        const int p0m = p0 % NSLOT;
        int xa[4][3], zoff[4];
        bool use[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int pi = 32 * (b0 + bb) + l32;
            const bool valid = pi < npix;
            const int pr = valid ? div_w(pi, invW) : 0;
            const int q = valid ? pi - pr * W : 0;
            zoff[bb] = 2 * (pi * HK + 32 * j + 4 * hi);     // byte offset of the lane's 4 channels
            use[bb] = valid && b0 + bb < b1;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                int sl = p0m + pr + r + NSLOT - 1;   // slot of row p0 + pr + r - 1 (>= -1)
                if (sl >= NSLOT) sl -= NSLOT;
                if (sl >= NSLOT) sl -= NSLOT;
                xa[bb][r] = WBYTES + sl * SLOT + q * PXB + hi * 16;
            }
        }

        f32x16 acc[4];
        // Full steps with 3 or 4 blocks run branch-free; other steps run all four slots
        // and drop the results they do not own.
        if (full && b1 - b0 == 4) {
            kloop<0xFu>(lds, wa, xa, acc, xr, tid, pf);
            epilogue<0xFu>(acc, zoff, use, zr, s1, s2);
        } else if (full && b1 - b0 == 3) {
            kloop<0x7u>(lds, wa, xa, acc, xr, tid, pf);
            epilogue<0x7u>(acc, zoff, use, zr, s1, s2);
        } else {
            kloop<0xFu>(lds, wa, xa, acc, xr, tid, pf);
            epilogue<0xFu>(acc, zoff, use, zr, s1, s2);
        }

        __syncthreads();                 // every wave is done reading the ring for step t
        if (next) store_rows(sn, pf);
        __syncthreads();
        n = nn;
        s = sn;
    }

    // Cross-lane sum through LDS, in the filter area (no longer read: the last step's
    // barriers have passed; 64 KB <= WBYTES).  st[f][tid] holds entry f of the lane's
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
           g.pw == 1 && g.W >= 2 && (TP + 1) * g.W * 8 <= PF * NT && g.P == g.H && g.Q == g.W;
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
