// conv3x3_c64.hip -- persistent 3x3 / stride 1 / pad 1 convolution with 64 input and 64
// output channels (the CBR page's N=256, 56x56, 64-channel workload), fused with the
// per-channel statistics of its output (the conv + genstats step of the CBR page's
// training forward, section 4.1).
//
// Each image is cut into steps of SP = 256 output pixels (8 blocks of 32) in NHWC order,
// regardless of where image rows begin, so that every SIMD has exactly two pixel blocks
// per full step.  One 512-thread workgroup per compute unit (two waves per SIMD) walks a
// contiguous range of the batch's steps (at most 256 ranges of near-equal length), so
// the grid fills the chip for any batch size and ranges may begin inside an image.
//   - Wave w computes output channels 32j .. 32j + 31, j = w / 4, and keeps that half of
//     the filter, 32 x 576 bf16, in registers (36 MFMA operand fragments, 144 VGPRs), so
//     LDS only serves input pixels.  Waves w and w + 4 share a SIMD and the same pixel
//     blocks: the SIMD holds both channel halves of its blocks.
//   - LDS holds a ring of input rows: the rows a step reads (its output rows +-1) and
//     the rows the next step adds, which stream in while the step computes.  Row h
//     (-1 <= h <= H) lives in slot (h + 1) % nslot; the padding rows -1 and H are zero
//     slots.  A slot holds W + 2 pixels of 64 channels (zero columns at both ends), 128
//     bytes each, whose eight 16-byte channel chunks are stored XOR-permuted by
//     (pixel / 2) % 8, so that 16 consecutive pixels of one fragment read hit 16 distinct
//     4-bank groups.
//   - Two staging buffers for a step's z (256 pixels x 128 bytes): the epilogues write
//     one; during the next step every wave stores a share of it as whole 1 KB runs of
//     pixel rows, which costs the memory pipeline a quarter of the cache-line
//     operations of storing straight from the MFMA layout.
// Input rows are copied from HBM straight into their slot with global-to-LDS loads (no
// register staging): a wave's load instruction moves 8 pixels, and each lane fetches the
// channel chunk that the permutation puts in its 16 bytes.  Each input row is read from
// HBM once and serves all nine taps.  Row loads and z stores are issued from inside the
// k-loops, one per k-step, rather than as a burst between steps.
//
// GEMM mapping: v_mfma_f32_32x32x16_bf16 with the filter as the A operand (32 output
// channels) and the input pixels as the B operand (32 pixels), so each lane ends up
// holding 4 consecutive output channels of one pixel.  The waves on SIMD s take blocks
// s and s + 4 of a step.
// The statistics are accumulated per lane in fp32 registers across the whole persistent
// loop, as sums of deviations (and their squares) from a per-lane shift -- the lane's own
// first value of each channel, so the sums do not cancel when a channel's mean is far
// from zero -- and combined across lanes and waves once at the end into one row of
// (count, mean, M2) per workgroup.
#include <hip/hip_ext.h>

#include "cbr_launch.h"
#include "cbr_persist.h"

namespace cbr {
namespace {

using persist::f32x16;
using persist::HK;
using persist::lds_u8;
using persist::make_rsrc;
using persist::NSIMD;
using persist::NT;
using persist::NW;
using persist::perm;
using persist::SP;
using persist::Staged;
using persist::STATS_BYTES;
using persist::STG_BYTES;
using persist::u32x2;

constexpr int HC = 64;                  // input channels
constexpr int PXB = HC * 2;             // bytes per staged input pixel (and per z pixel)
static_assert(PXB == persist::PXB, "input and output pixels have the same size");
constexpr int MAXW = 56;
constexpr int KSTEPS = 36;              // 9 taps x 4 chunks of 16 input channels
constexpr int FILTER_BYTES = HK * 72 * 16;    // the filter, staged once through LDS
// Row loads per wave per step: a step adds at most ceil(SP / W) input rows of W / 8
// loads each, i.e. at most SP / 8 + W / 8 <= 39 loads over the 8 waves.
constexpr int LPW = 5;
static_assert(NW * LPW >= SP / 8 + MAXW / 8, "row loads per step");

struct HaloParams {
    const uint16_t *x;
    const uint16_t *w;
    uint16_t *z;
    float *partials;       // [gridDim.x][2][64]
    int N, H, W;
    int slot_bytes;        // (W + 2) * PXB
    int nslot;             // ring slots: >= the rows a step reads plus the rows the next adds
    uint32_t mW;           // ceil(2^32 / W): v / W == mulhi(v, mW) for v < 2^32 / W
};

__device__ __forceinline__ int div_w(int v, uint32_t mW) { return (int)__umulhi((uint32_t)v, mW); }

// Input pixels are permuted like staged z pixels (perm, with row_flip): channel chunk c
// of pixel u of input row h is stored at position c ^ perm(u) ^ row_flip(h).

// The input-row permutation continues across rows as if the rows were one run of pixels:
// pixel u of row h is permuted like pixel u + (h + 1) W of one long row, i.e. by
// perm(u) ^ row_flip(h), the flip 4 ((h + 1) W / 8 mod 2) (W a multiple of 8).  A pixel
// block that spans two rows then reads 32 consecutive permutation positions, as one
// inside a row does; with a plain per-row permutation the two rows' positions repeat and
// every read of such a block takes twice as long.
__device__ __forceinline__ int row_flip(int h, int ipr) { return (((h + 1) * ipr) & 1) << 2; }

// Per pixel block: LDS address of the lane's staged pixel q in the slot of tap row r
// (rb[r]), and the lane's chunk permutation of pixels q + sx, pre-shifted and with the
// lane's k-half folded in (cx[f][sx] = (hi ^ perm(q + sx) ^ row_flip(h)) << 4, f = 1 for
// the middle tap row, whose flip differs from the other two): the fragment of tap
// (r, sx), 16-channel chunk kc is at rb[r] + 128 sx + ((32 * kc) ^ cx[r == 1][sx]).
struct BlockAddr {
    int rb[3];
    int cx[2][3];
};

// LDS fragment reads in inline assembly, with explicit waits.  While global-to-LDS loads
// are in flight the compiler waits for every outstanding LDS read before each use
// (lgkmcnt(0)), which would drain the read-ahead below at every k-step; reads from
// assembly are outside its tracking, and the k-loop waits for exactly the reads it
// needs.  LDS reads complete in order, so "at most n outstanding" means all but the n
// newest are done (other LDS or scalar memory operations only add to the count).
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr)
{
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}

// The fragment about to be used is tied to the wait, so that its use cannot be
// scheduled above it.
template <int N>
__device__ __forceinline__ void lds_wait(bf16x8 &x)
{
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}

// The 36 k-steps of one pixel block for the wave's 32 output channels: per k-step one
// LDS fragment read and one MFMA, the filter fragment from registers.  Fragments are read
// KD - 2 k-steps ahead, each issued after the MFMA of the k-step before it.
// side(integral_constant<T>) issues the memory instructions that belong to k-step T.
template <typename Side>
struct KLoop {
    static constexpr int KD = 4;
    const bf16x8 (&wf)[KSTEPS];
    const BlockAddr &ba;
    f32x16 &acc;
    Side &side;
    bf16x8 xf[KD];

    // Fragment read of k-step T (tap T / 4 = (r, sx), chunk T % 4) into set T % KD.
    template <int T>
    __device__ __forceinline__ void read()
    {
        constexpr int tap = T >> 2, kc = T & 3, r = tap / 3, sx = tap - 3 * r;
        xf[T % KD] = lds_read16<128 * sx>(ba.rb[r] + ((32 * kc) ^ ba.cx[r == 1][sx]));
    }

    template <int T>
    __device__ __forceinline__ void step()
    {
        // the reads of k-steps T + 1 .. min(T + KD - 2, 35) may stay in flight
        constexpr int newer = (KSTEPS - 1 - T) < (KD - 2) ? (KSTEPS - 1 - T) : (KD - 2);
        lds_wait<newer>(xf[T % KD]);
        __builtin_amdgcn_sched_barrier(0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[T], xf[T % KD], T == 0 ? f32x16{} : acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // The read for k-step T + KD - 1 goes after MFMA T, into the fragment set of MFMA
        // T - 1, which has finished (MFMA T depends on it).  MFMA T's own fragment is kept
        // live past the read, so that neither the read nor its address arithmetic reuses
        // registers the in-flight MFMA still reads (such a write waits for the MFMA).
        if constexpr (T + KD - 1 < KSTEPS) read<T + KD - 1>();
        asm volatile("" ::"v"(xf[T % KD]));
        side(std::integral_constant<int, T>{});
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (T + 1 < KSTEPS) step<T + 1>();
    }

    template <int T>
    __device__ __forceinline__ void prefetch()
    {
        read<T>();
        if constexpr (T + 1 < KD - 1) prefetch<T + 1>();
    }

    __device__ __forceinline__ void run()
    {
        prefetch<0>();
        step<0>();
    }
};

__global__ __launch_bounds__(NT, 1) void conv3x3_c64_stats_kernel(HaloParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int simd = wave & (NSIMD - 1), j = wave >> 2;
    const int H = p.H, W = p.W, SLOT = p.slot_bytes, NSLOT = p.nslot;
    const uint32_t mW = p.mW;
    const int HW = H * W;
    const int spi = (HW + SP - 1) / SP;                       // steps per image
    // This workgroup's steps: a contiguous range [t0, t1) of the N * spi steps of the batch
    // in order (step s of image n is step n * spi + s), spread evenly over the grid, so
    // every CU has work whatever N is and ranges may start inside an image.
    const long tot = (long)p.N * spi;
    const int t0 = (int)(tot * blockIdx.x / gridDim.x), t1 = (int)(tot * (blockIdx.x + 1) / gridDim.x);
    const int n_first = t0 / spi, s_first = t0 - n_first * spi;
    const int hi = lane >> 5;                                 // k-half of the MFMA operands
    const int l32 = lane & 31;
    const int ipr = W / 8;                                    // 8-pixel load instructions per row
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_u8 *)lds;
    uint8_t *const stg0 = lds + NSLOT * SLOT;                 // two step staging buffers
    // Input rows -1 .. rows0 - 2 are the first step's: its output rows 0 .. last +- 1.
    const int rows0 = div_w(min(SP, HW) - 1, mW) + 3;

    // Load k (pixels 8k .. 8k + 7) of input row h (-1 <= h <= H) of image n into its slot:
    // an image row by a global-to-LDS load, the padding rows as zeros.  Lane l moves pixel
    // 8k + l/8, position l % 8, which holds channel chunk (l % 8) ^ perm(1 + 8k + l/8).
    auto stage_part = [&](int n, int h, int k, int ln) {
        const int dst = ((h + 1) % NSLOT) * SLOT + (1 + 8 * k) * PXB;   // wave-uniform
        if (h >= 0 && h < H) {
            const int u = 1 + 8 * k + (ln >> 3);
            const uint16_t *src =
                p.x + ((size_t)(n * H + h) * W + 8 * k + (ln >> 3)) * HC + (((ln & 7) ^ perm(u) ^ row_flip(h, ipr)) * 8);
            __builtin_amdgcn_global_load_lds((const void *)src, (lds_u8 *)lds + dst, 16, 0, 0);
        } else {
            *(u32x4 *)(lds + dst + ln * 16) = u32x4{0, 0, 0, 0};
        }
    };
    // Rows h0 .. h0 + nrows - 1 of image n: load gi (row gi / ipr, pixels 8 (gi % ipr) ..)
    // is issued by wave gi % 8.  gi / ipr == 8 gi / W.
    auto stage_rows = [&](int n, int h0, int nrows) {
        for (int gi = wave; gi < nrows * ipr; gi += NW) {
            const int ri = div_w(8 * gi, mW);
            stage_part(n, h0 + ri, gi - ri * ipr, lane);
        }
    };
    // A step's 1 KB z runs q = wave % 4 + 4 (4 half + k), k < 4, go out in two halves of
    // four: half 0 from the waves of channel half 0, half 1 from the others.
    // load_staged reads a half of staging buffer buf into sd, with reads in assembly that
    // the compiler does not track (its own waits for them, at the stores inside the first
    // k-loop, would count only these four reads and drain the k-loop's read-ahead).  The
    // k-loop's first wait (all but the two newest LDS operations done) covers them before
    // its stores, LDS operations completing in order; elsewhere staged_wait precedes the
    // stores.
    auto load_staged = [&](Staged &sd, int buf, int half, int ln) {
        const uint32_t sb = lbase + (uint32_t)(NSLOT * SLOT + buf * STG_BYTES);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int px = 8 * (simd + NSIMD * (4 * half + k)) + (ln >> 3);   // < SP
            const uint32_t a = sb + px * PXB + (((ln & 7) ^ perm(px)) << 4);
            asm volatile("ds_read_b128 %0, %1" : "=v"(sd.d[k]) : "v"(a) : "memory");
        }
    };
    auto staged_wait = [](Staged &sd) {
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(sd.d[0]), "+v"(sd.d[1]), "+v"(sd.d[2]), "+v"(sd.d[3]));
    };
    // Runs q >= nq lie past the end of zr (npix * 128 = nq * 1024 bytes): the buffer
    // store drops them, so no condition is needed.  The stores stream (nt) and write
    // through to the device's coherence point (sc1): z is not read again in this kernel,
    // and lines left dirty in L2 would have to be written back when the kernel ends,
    // between it and the next kernel of the step.
    constexpr int Z_POLICY = 2 | 16;   // nt | sc1
    auto store_staged = [&](const Staged &sd, int half, int k, int ln) {
        const int q = simd + NSIMD * (4 * half + k);
        __builtin_amdgcn_raw_buffer_store_b128(sd.d[k], sd.zr, q * 1024 + ln * 16, 0, Z_POLICY);
    };

    // The filter half into registers, through LDS, past the first step's ring slots (in
    // slots the first k-loop has not loaded yet and in the staging buffers).  Filter row r
    // (output channel; KRSC: 72 chunks of 16 bytes, 1152 bytes, nine cache lines) has its
    // chunks in groups of eight, one cache line each.  Global-to-LDS load i moves line
    // i % 9 of rows 8 (i / 9) .. + 7: lane l takes row 8 (i / 9) + l / 8 and chunk
    // 8 (i % 9) + fsw(row, l % 8), so each load reads eight whole lines, and LDS
    // position 16 l of load i holds that chunk.  fsw(r, q) = q ^ (r % 8) ^ ((r / 8) % 2)
    // spreads the fragment reads below over the banks: their 16 lanes of rows
    // 8b .. 8b + 15 and one chunk land in 16 distinct 16-byte bank slots.  Fragment t of
    // lane (l32, hi) is output channel 32j + l32, tap t / 4, input channels
    // 16 (t % 4) + 8 hi .. + 7: chunk 8 (t / 4) + 2 (t % 4) + hi.  When the range starts
    // at an image's first step, that step's rows stream into slots 0 .. rows0 - 1
    // meanwhile, and the filter sits past them; a range starting inside an image stages
    // the filter at the start of LDS first and its first step's rows once the filter is
    // in registers.
    const bool at_start = s_first == 0;
    const int F = at_start ? rows0 * SLOT : 0;
    for (int i = wave; i < 72; i += NW) {
        const int row = 8 * (i / 9) + (lane >> 3);
        const int ch = 8 * (i % 9) + ((lane & 7) ^ (row & 7) ^ ((row >> 3) & 1));
        __builtin_amdgcn_global_load_lds((const void *)(p.w + ((size_t)row * 72 + ch) * 8), (lds_u8 *)lds + F + i * 1024,
                                         16, 0, 0);
    }
    const int zrows = at_start ? rows0 : 0;   // slots whose padding columns are zeroed now
    for (int c = tid; c < zrows * 16; c += NT) {
        const int slot = c >> 4, col = (c & 8) ? W + 1 : 0;
        *(u32x4 *)(lds + slot * SLOT + col * PXB + (c & 7) * 16) = u32x4{0, 0, 0, 0};
    }
    if (at_start && t1 > t0) stage_rows(n_first, -1, rows0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    bf16x8 wf[KSTEPS];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
        wf[t] = *(const bf16x8 *)(lds + F + ((4 * j + (l32 >> 3)) * 9 + (t >> 2)) * 1024 +
                                  (8 * (l32 & 7) + ((2 * (t & 3) + hi) ^ (l32 & 7) ^ ((l32 >> 3) & 1))) * 16);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // the filter area is free again
    // The padding columns of the other slots zeroed (the k-loops' row loads fill the
    // other columns).
    for (int c = zrows * 16 + tid; c < NSLOT * 16; c += NT) {
        const int slot = c >> 4, col = (c & 8) ? W + 1 : 0;
        *(u32x4 *)(lds + slot * SLOT + col * PXB + (c & 7) * 16) = u32x4{0, 0, 0, 0};
    }
    if (!at_start) {
        // input rows ofr - 1 .. olr + 1 of the first step's first and last output rows
        const int a = s_first * SP, npix = min(SP, HW - a);
        const int ofr = div_w(a, mW), olr = div_w(a + npix - 1, mW);
        stage_rows(n_first, ofr - 1, olr - ofr + 3);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // Per-lane running statistics (layout: see epilogue).
    float c[8], s1[8], s2[8], cnt = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        c[i] = 0.f;
        s1[i] = 0.f;
        s2[i] = 0.f;
    }
    bool first = true;   // wave-uniform: the wave's first pixel block sets the shifts

    Staged prev;          // the previous step, staged in buffer pbuf
    prev.nq = 0;
    prev.zr = make_rsrc(p.z, 0);   // nothing staged yet: every store is dropped
    int pbuf = 1;
    constexpr int DMA_T0 = 6;                                 // k-step of the first row load
    static_assert(DMA_T0 + LPW <= KSTEPS, "the row loads fit in one k-loop");
    static_assert(2 * 4 * NSIMD * 1024 == STG_BYTES, "two halves of runs cover a step");
    int n = n_first, s = s_first;   // image and step within it of step t
    for (int t = t0; t < t1; ++t, ++s) {
        if (s == spi) {
            // The next image: every wave is past the last step's reads; restage its first
            // rows.
            ++n;
            s = 0;
            stage_rows(n, -1, rows0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        const bool more = t + 1 < t1 && s + 1 < spi;   // the range's next step is in this image
        // Opaque per-step copy of the lane id: lane-derived addresses are recomputed
        // each step instead of being hoisted into registers held through the k-loops.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int l32s = ln & 31, his = ln >> 5;
        const int a = s * SP;                               // first pixel of the step
        const int npix = min(SP, HW - a);
        const int nblk = (npix + 31) >> 5;                  // <= 8
        const int nb = (simd < nblk) + (simd + NSIMD < nblk);
        const bool full = npix == 32 * nblk;                // every pixel block complete
        const int ofr = div_w(a, mW);                       // first output row of the step
        const int olr = div_w(a + npix - 1, mW);            // last output row
        const int fslot = ofr % NSLOT;                      // slot of input row ofr - 1
        // The next step's new input rows olr + 2 .. olr1 + 1 (none after the image's
        // last step) stream into their slots: load gi of them (row olr + 2 + gi / ipr,
        // pixels 8 (gi % ipr) ..) goes to wave gi % 8 at k-step DMA_T0 + gi / 8.  The
        // rows below H are contiguous in x, so load gi reads bytes 1024 gi .. of them;
        // row H (the bottom padding) is written as zeros.
        int nload = 0, nmem = 0;
        if (more) {
            const int a1 = a + SP;
            const int olr1 = div_w(a1 + min(SP, HW - a1) - 1, mW);
            nload = (olr1 - olr) * ipr;
            nmem = max(0, min(olr1, H - 2) - olr) * ipr;
        }
        const int slot_a = (olr + 3) % NSLOT;                // slot of input row olr + 2
        const uint16_t *const xa = p.x + ((size_t)n * H + olr + 2) * W * HC;
        auto row_part = [&](auto tc, int lt) {
            constexpr int t = decltype(tc)::value - DMA_T0;
            const int gi = wave + NW * t;                   // wave-uniform
            if (gi < nload) {
                const int ri = div_w(8 * gi, mW);
                const int k = gi - ri * ipr;
                int sl = slot_a + ri;
                if (sl >= NSLOT) sl -= NSLOT;
                const int dst = sl * SLOT + (1 + 8 * k) * PXB;
                if (gi < nmem) {
                    // lane l: pixel 8k + l/8, position l % 8, which holds channel chunk
                    // (l % 8) ^ perm(1 + 8k + l/8) ^ row_flip(h)
                    //   = (l % 8) ^ ((1 + l/8) / 2) ^ 4 (k % 2) ^ row_flip(h)
                    const int l8 = lt >> 3;
                    const int off = (l8 * HC + (((lt & 7) ^ ((1 + l8) >> 1)) << 3)) ^
                                    (((k & 1) << 5) ^ (row_flip(olr + 2 + ri, ipr) << 3));
                    __builtin_amdgcn_global_load_lds((const void *)(xa + gi * 512 + off), (lds_u8 *)lds + dst,
                                                     16, 0, 0);
                } else {
                    *(u32x4 *)(lds + dst + lt * 16) = u32x4{0, 0, 0, 0};
                }
            }
        };
        const int cbuf = pbuf ^ 1;
        uint8_t *const stg = stg0 + cbuf * STG_BYTES;
        // The previous step's z: channel half 0's waves store the first half of its
        // runs, the others the second half.
        load_staged(prev, pbuf, j, ln);
        if (nb == 0) {   // only in an image's last step (no row loads): no k-loop
            staged_wait(prev);
            for (int k = 0; k < 4; ++k) store_staged(prev, j, k, ln);
        }
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            if (bb >= nb) break;
            const int px = 32 * (simd + NSIMD * bb) + l32s;   // pixel within the step
            const bool use = px < npix;
            const int pi = a + (use ? px : 0);
            const int pr = div_w(pi, mW);
            const int q = pi - pr * W;
            BlockAddr ba;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                int sl = fslot + (pr - ofr) + r;            // slot of input row pr + r - 1
                if (sl >= NSLOT) sl -= NSLOT;
                ba.rb[r] = (int)lbase + sl * SLOT + q * PXB;
            }
#pragma unroll
            for (int sx = 0; sx < 3; ++sx) {
                // rows pr - 1 and pr + 1 share a flip; row pr's differs when W / 8 is odd
                ba.cx[0][sx] = (his ^ perm(q + sx) ^ row_flip(pr - 1, ipr)) << 4;
                ba.cx[1][sx] = ba.cx[0][sx] ^ ((ipr & 1) << 6);
            }

            f32x16 acc;
            if (bb == 0) {
                // k-steps 2..5: this wave's half of the previous step's z runs (its LDS
                // reads have landed by then); 6 .. 6 + LPW - 1: the row loads
                auto side = [&](auto tc) {
                    constexpr int T = decltype(tc)::value;
                    // an opaque lane id per k-step keeps each instruction's address
                    // computation at its k-step instead of in registers held from the start
                    int lt = ln;
                    asm volatile("" : "+v"(lt));
                    if constexpr (T >= 2 && T < 6) {
                        store_staged(prev, j, T - 2, lt);
                    } else if constexpr (T >= DMA_T0 && T < DMA_T0 + LPW) {
                        row_part(tc, lt);
                    }
                };
                KLoop<decltype(side)>{wf, ba, acc, side}.run();
            } else {
                auto side = [](auto) {};
                KLoop<decltype(side)>{wf, ba, acc, side}.run();
            }
            if (full)
                persist::epilogue<false>(acc, use, true, first, stg, px, j, his, c, s1, s2, cnt);
            else
                persist::epilogue<true>(acc, use, (px ^ 16) < npix, first, stg, px, j, his, c, s1, s2, cnt);
            first = false;
        }

        // The staged rows must have landed before any wave reads them: wait for this
        // wave's loads, then the barrier publishes every wave's.  The barrier also
        // frees the slots this step read for the steps after it, and publishes this
        // step's staged z.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        prev.nq = npix / 8;
        prev.zr = make_rsrc(p.z + ((size_t)n * HW + a) * HK, npix * HK * 2);
        pbuf = cbuf;
    }
    load_staged(prev, pbuf, j, lane);
    staged_wait(prev);
    for (int k = 0; k < 4; ++k) store_staged(prev, j, k, lane);
    __syncthreads();   // every wave is done with the staging buffers and the ring

    persist::store_stat_row(lds, c, s1, s2, cnt, p.partials, blockIdx.x, gridDim.x);
}

}  // namespace

// Ring slots: the input rows of a step and the rows the next one adds, ofr(s) - 1 ..
// olr(s + 1) + 1, number at most floor((2 SP - 1) / W) + 4 (the output rows of 2 SP
// consecutive pixels span at most floor((2 SP - 1) / W) + 2 rows).
int halo_nslot(const ConvGeom &g) { return (2 * SP - 1) / g.W + 4; }

// Input rows of an image's first step: -1 .. its last output row + 1.
int halo_rows0(const ConvGeom &g) { return (std::min(SP, g.H * g.W) - 1) / g.W + 3; }

size_t halo_lds_bytes(const ConvGeom &g)
{
    const size_t slot = (size_t)(g.W + 2) * PXB;
    return std::max({halo_nslot(g) * slot + 2 * STG_BYTES, halo_rows0(g) * slot + FILTER_BYTES,
                     (size_t)STATS_BYTES});
}

bool halo_eligible(const ConvGeom &g)
{
    if (!(g.C == HC && g.K == HK && g.R == 3 && g.S == 3 && g.sh == 1 && g.sw == 1 && g.ph == 1 && g.pw == 1 &&
          g.W >= 8 && g.W <= MAXW && g.W % 8 == 0 && g.P == g.H && g.Q == g.W && g.H >= 1))
        return false;
    // pixel indices of an image (and of the step past its end) must stay below 2^32 / W
    // for the multiply-high division, and in int range
    const uint64_t hw = (uint64_t)g.H * g.W + SP;
    return hw * g.W < (1ull << 32) && halo_lds_bytes(g) <= (size_t)HALO_MAX_LDS;
}

int halo_grid(const ConvGeom &g)
{
    const long steps = (long)g.N * ((g.H * g.W + SP - 1) / SP);
    return (int)std::min<long>(steps, HALO_MAX_GRID);
}

hipError_t launch_conv3x3_c64_stats(const ConvGeom &g, const uint16_t *x, const uint16_t *w, uint16_t *z,
                                    float *partials, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    static_assert(((2 * SP - 1) / MAXW + 4) * (MAXW + 2) * PXB + 2 * STG_BYTES <= HALO_MAX_LDS,
                  "the ring for W = MAXW fits");
    const uint32_t mW = (uint32_t)(((1ull << 32) + g.W - 1) / g.W);
    HaloParams prm{x, w, z, partials, g.N, g.H, g.W, (g.W + 2) * PXB, halo_nslot(g), mW};
    const size_t lds = halo_lds_bytes(g);
    const hipError_t e = raise_lds_limit((const void *)conv3x3_c64_stats_kernel, (int)lds);
    if (e != hipSuccess) return e;
    const dim3 grid(halo_grid(g)), block(NT);
    if (e0 || e1)
        hipExtLaunchKernelGGL(conv3x3_c64_stats_kernel, grid, block, (uint32_t)lds, st, e0, e1, 0, prm);
    else
        conv3x3_c64_stats_kernel<<<grid, block, lds, st>>>(prm);
    return hipGetLastError();
}

}  // namespace cbr
