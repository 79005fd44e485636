// conv_c3s2.hip -- persistent first-layer convolution (3 input channels, stride 2, up
// to 7x8 taps, 64 output channels) fused with the per-channel statistics of its output:
// the training forward's conv + genstats step (CBR page, section 4.1) for the network's
// input layer.
//
// With 3 channels a pixel is 6 bytes, so a generic implicit GEMM would gather element by
// element.  Here input pixels are widened to 4 channels (8 bytes, the fourth zero) and
// the filter to [64][R][8][4] (taps s >= S and channel 3 zero), so that for a fixed tap
// row r the 16 values of one MFMA k-step are four consecutive input pixels x 4 channels
// and, with stride 2, the 8 values a lane needs for output column q are one aligned
// 16-byte LDS read at widened pixel 2q + s0 (2R k-steps, R*32 reduction slots of which
// R*S*3 are live).
// Schedule:
//   - One 512-thread workgroup per CU walks a contiguous range of the batch's steps of
//     128 output pixels (4 blocks of 32, NHWC order, starting anywhere in a row).
//   - Wave specialisation: waves 0..3, one per SIMD, keep the whole widened filter in
//     registers (4R fragments) and compute their block of each step, both channel halves,
//     into an LDS result buffer (fp32); waves 4..7 turn the previous step's results into
//     statistics and bf16 z, and load and widen the input rows later steps add.
//   - LDS holds a ring of widened input rows (zero columns on both sides; rows outside
//     the image are zero rows) in which consecutive images' rows follow each other, and
//     two result buffers; one barrier per step hands rows and results over.
//   - The statistics are kept per lane as shifted sums and combined once at the end into
//     one (count, mean, M2) row per workgroup.
#include <type_traits>

#include "cbr_launch.h"
#include "cbr_persist.h"

namespace cbr {
namespace {

using namespace persist;

constexpr int MAXR = 7;    // filter rows

struct C3PParams {
    const uint16_t *x;      // N x H x W x 3
    const uint16_t *w;      // 64 x R x S x 3 (KRSC)
    uint16_t *z;            // N x P x Q x 64
    float *partials;        // [gridDim.x][2][64] means and M2, then [gridDim.x] counts
    int N, H, W, R, S, ph, pw, P, Q;
    int slot_bytes;         // LW * 8: widened pixels per staged row, zero columns included
    int nslot;              // ring slots
    int vpi;                // input rows an image spans: 2 (P - 1) + R
    uint32_t mQ, mG;        // ceil(2^32 / Q), ceil(2^32 / (W / 8)): multiply-high divisions
};

// v / d for the divisor d whose magic m = ceil(2^32 / d) (truncated to 32 bits) is given:
// exact for v < 2^32 / d; d = 1 has m = 0 and returns v.
__device__ __forceinline__ int div_m(int v, uint32_t m) { return m ? (int)__umulhi((uint32_t)v, m) : v; }

// Workgroup barrier over LDS only: every wave's LDS operations have completed when any
// wave passes it; global stores stay in flight (nothing in the kernel reads what they
// write, and their data was read from registers when they were issued).  The memory
// clobbers keep the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A block's fragment reads are inline assembly issued together, and each MFMA waits
// (explicit lgkmcnt, tied to its fragment) for exactly its own read: left to itself the
// compiler placed every read right before its MFMA behind a full wait, one LDS latency
// per MFMA.  LDS operations complete in order, so "at most n outstanding" means all but
// the n newest are done (scalar memory operations only add to the count).
__device__ __forceinline__ bf16x8 lds_rd(uint32_t addr)
{
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
template <int N>
__device__ __forceinline__ void lds_wait(bf16x8 &x)
{
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
template <int R, int T>
__device__ __forceinline__ void mfma_chain(f32x16 &acc, const bf16x8 (&wf)[2 * R], bf16x8 (&xf)[2 * R])
{
    lds_wait<2 * R - 1 - T>(xf[T]);
    __builtin_amdgcn_sched_barrier(0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[T], xf[T], acc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (T + 1 < 2 * R) mfma_chain<R, T + 1>(acc, wf, xf);
}

// Eight pixels of an input row: 48 bytes of x (three 16-byte loads).
struct Piece {
    u32x4 a, b, d;
};

constexpr int WSP = 128;                 // output pixels per step: 4 blocks of 32, one per SIMD
constexpr int NMW = NSIMD;               // MFMA waves 0..3, wave w on SIMD w
constexpr int NEW = NSIMD;               // epilogue waves 4..7, wave w on SIMD w % 4
constexpr int NET = NEW * 64;            // epilogue threads
constexpr int PPT = 2;                   // row pieces per epilogue thread and step, at most
constexpr int ACC_ROW = HK * 4;          // bytes of one pixel's 64 fp32 results
constexpr int ACC_BYTES = WSP * ACC_ROW; // one step's results
constexpr int EST_BYTES = NEW * 8 * 17 * 4;   // the end-of-kernel combination area

// Results of one step in LDS: pixel px's 64 fp32 values in a 256-byte row, 16-byte chunk
// ci (channels 4ci .. 4ci + 3) at position ci ^ (px % 16), so that both the MFMA waves'
// writes (16 pixels, one chunk each) and the epilogue waves' reads (2 pixels, 8 chunks
// each) cover all 64 banks.
__device__ __forceinline__ int acc_off(int px, int ci) { return px * ACC_ROW + ((ci ^ (px & 15)) << 4); }

// MFMAs T .. 2R - 1 of a chain whose fragments have all landed.
template <int R, int T>
__device__ __forceinline__ void mfma_chain_in(f32x16 &acc, const bf16x8 (&wf)[2 * R], const bf16x8 (&xf)[2 * R])
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[T], xf[T], acc, 0, 0, 0);
    if constexpr (T + 1 < 2 * R) mfma_chain_in<R, T + 1>(acc, wf, xf);
}

// R (the filter's rows) is a template parameter: the k-loops are then straight-line code
// (2R fragment reads, then 4R MFMAs), with no run-time guards between the reads.
//
// Wave specialisation.  Waves 0..3 (one per SIMD) hold the whole widened filter in
// registers and do nothing but the MFMAs of their pixel block of each step (both channel
// halves), writing the fp32 results to one of two LDS result buffers.  Waves 4..7 (the
// other wave of each SIMD) do everything else: during step s they turn step s - 1's
// results into statistics and bf16 z (stored to global memory straight from registers,
// whole 1 KB runs), load the input rows step s + 2 adds and widen those of step s + 1.
// One barrier per step hands rows and results over.  The epilogue work of one wave then
// runs beside the MFMAs of the other on each SIMD, where with every wave doing both the
// two phases alternated.
template <int R>
__global__ __launch_bounds__(NT, 1) void conv_c3s2_ws_kernel(C3PParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool mw = wave < NMW;
    const int hi = lane >> 5, l32 = lane & 31;
    const int H = p.H, W = p.W, Q = p.Q, SB = p.slot_bytes, NSLOT = p.nslot, VPI = p.vpi;
    const int PQ = p.P * Q;
    const int spi = (PQ + WSP - 1) / WSP;                     // steps per image
    // This workgroup's steps: a contiguous range [t0, t1) of the N * spi steps of the batch
    // (step s of image n is step n * spi + s), spread evenly over the grid.
    const long tot = (long)p.N * spi;
    const int t0 = (int)(tot * blockIdx.x / gridDim.x), t1 = (int)(tot * (blockIdx.x + 1) / gridDim.x);
    const int gpr = W / 8;                                    // 8-pixel pieces per input row
    constexpr int nks = 2 * R;
    uint8_t *const accb = lds + NSLOT * SB;                   // two result buffers

    // The ring: input row h of the range's image i (i = 0 for the image of step t0) is
    // virtual row v = i * VPI + h + ph, VPI = 2 (P - 1) + R being the rows an image spans,
    // and lives in slot v % nslot.  Consecutive images' rows follow each other, so the
    // first rows of the next image load during the last step of the previous one.
    // Piece g of input row h of image n (zeros outside the image), and its widened store
    // at dst (pixel u of a row at byte (pw + u) * 8 of its slot, so dst = slot base +
    // (pw + 8 g) * 8).
    auto load_piece = [&](int n, int h, int g) {
        Piece r;
        if (h >= 0 && h < H) {
            const u32x4 *src = (const u32x4 *)(p.x + (((size_t)n * H + h) * W + 8 * g) * 3);
            r.a = src[0];
            r.b = src[1];
            r.d = src[2];
        } else {
            r.a = r.b = r.d = u32x4{0u, 0u, 0u, 0u};
        }
        return r;
    };
    auto store_piece_at = [&](uint8_t *dst, const Piece &r) {
        const uint32_t v[12] = {r.a[0], r.a[1], r.a[2], r.a[3], r.b[0], r.b[1], r.b[2], r.b[3], r.d[0], r.d[1], r.d[2], r.d[3]};
        // bf16 value t of the piece is half t % 2 of word t / 2; pixel e is values 3e .. 3e + 2
        auto half = [&](int t) { return (v[t >> 1] >> (16 * (t & 1))) & 0xffffu; };
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *(u32x2 *)(dst + e * 8) = u32x2{half(3 * e) | (half(3 * e + 1) << 16), half(3 * e + 2)};
    };

    // The zero columns of every slot (left of the image and right of it, up to the last
    // widened pixel a read can reach).
    {
        const int lw = SB / 8, nz = lw - W;
        for (int i = tid; i < NSLOT * nz; i += NT) {
            const int sl = i / nz, c = i - sl * nz;
            const int col = c < p.pw ? c : W + c;
            *(u32x2 *)(lds + sl * SB + col * 8) = u32x2{0u, 0u};
        }
    }
    int n = t0 / spi, s = t0 - n * spi, img = 0;             // image, its step, its index in the range
    if (t1 > t0) {
        // the first step's input rows 2 ofr - ph .. 2 olr - ph + R - 1, by every thread
        const int a = s * WSP, npix = min(WSP, PQ - a);
        const int ofr = div_m(a, p.mQ), olr = div_m(a + npix - 1, p.mQ);
        const int nrows = 2 * (olr - ofr) + R;
        for (int i = tid; i < nrows * gpr; i += NT) {
            const int ri = div_m(i, p.mG);
            const int g = i - ri * gpr;
            store_piece_at(lds + ((2 * ofr + ri) % NSLOT) * SB + (p.pw + 8 * g) * 8, load_piece(n, 2 * ofr - p.ph + ri, g));
        }
    }

    // The widened filter [64][R][8][4] (element ((k R + r) 8 + s) 4 + c: taps s >= S and
    // channel 3 zero), built by every thread from the KRSC filter in the second result
    // buffer, which the MFMA waves first write in the range's second step: by then every
    // MFMA wave has passed the first step's barrier, so has its fragments.  One 8-byte
    // group (k, r, s) per iteration.
    {
        // every thread's groups gathered first (their loads all in flight), then stored
        constexpr int NG = (HK * R * 8 + NT - 1) / NT;
        uint8_t *const wl = accb + ACC_BYTES;
        uint32_t lo[NG], hv[NG];
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int i = tid + NT * u, s8 = i & 7, kr = i >> 3;   // kr = k R + r
            lo[u] = 0;
            hv[u] = 0;
            if (i < HK * R * 8 && s8 < p.S) {
                const uint16_t *src = p.w + ((size_t)kr * p.S + s8) * 3;
                lo[u] = (uint32_t)src[0] | ((uint32_t)src[1] << 16);
                hv[u] = src[2];
            }
        }
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int i = tid + NT * u;
            if (i < HK * R * 8) *(u32x2 *)(wl + i * 8) = u32x2{lo[u], hv[u]};
        }
    }
    __syncthreads();

    // The step sequence, the same for both kinds of wave (each passes one barrier per step).
    struct StepIt {
        int n, s, img;
    };
    StepIt it0{n, s, img};

    if (mw) {
        // MFMA waves: the widened filter, both channel halves.  Fragment t of half j: lane
        // (l32, hi) holds output channel 32j + l32, tap row t / 2, taps 4 (t % 2) + 2 hi
        // and + 1, four channels each: 16 bytes of the widened filter.
        const int msimd = wave;
        const uint8_t *const wl = accb + ACC_BYTES;
        bf16x8 w0[nks], w1[nks];
#pragma unroll
        for (int t = 0; t < nks; ++t) {
            w0[t] = *(const bf16x8 *)(wl + ((l32 * R + (t >> 1)) * 32 + 16 * (t & 1) + 8 * hi) * 2);
            w1[t] = *(const bf16x8 *)(wl + (((32 + l32) * R + (t >> 1)) * 32 + 16 * (t & 1) + 8 * hi) * 2);
        }
        // every read of it done before the step loop's counted waits
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        int cbuf = 0;
        StepIt it = it0;
        for (int t = t0; t < t1; ++t, ++it.s) {
            if (it.s == spi) {
                ++it.n;
                ++it.img;
                it.s = 0;
            }
            const int a = it.s * WSP;                           // first pixel of the step
            const int npix = min(WSP, PQ - a);
            const int ofr = div_m(a, p.mQ);
            // Block msimd of the step: pixels past the step compute the step's first pixel.
            const int px = 32 * msimd + l32;
            const int pi = a + (px < npix ? px : 0);
            const int pr = div_m(pi, p.mQ);
            const int q = pi - pr * Q;
            // tap row r of output row pr reads input row 2 pr - ph + r: virtual row
            // img VPI + 2 pr + r
            int sl0 = (it.img * VPI + 2 * ofr) % NSLOT + 2 * (pr - ofr);
            while (sl0 >= NSLOT) sl0 -= NSLOT;
            const uint32_t lb = (uint32_t)(uintptr_t)(lds_u8 *)lds + 16 * q + 16 * hi;
            bf16x8 xf[nks];
#pragma unroll
            for (int tt = 0; tt < nks; ++tt) {
                int sl = sl0 + (tt >> 1);
                if (sl >= NSLOT) sl -= NSLOT;
                xf[tt] = lds_rd(lb + sl * SB + 32 * (tt & 1));
            }
            f32x16 acc0, acc1;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                acc0[v] = 0.f;
                acc1[v] = 0.f;
            }
            // Channel half 0 as the fragments land, then half 1 from the same fragments;
            // half 0's results are written out behind half 1's first MFMAs.
            mfma_chain<R, 0>(acc0, w0, xf);
            mfma_chain_in<R, 0>(acc1, w1, xf);   // placed by the scheduler up to the barrier below
            // acc_j[4g + e] is channel 32j + 8g + 4hi + e of pixel px: chunk 8j + 2g + hi
            uint8_t *ab = accb + cbuf * ACC_BYTES;
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(f32x4 *)(ab + acc_off(px, 2 * g + hi)) =
                    f32x4{acc0[4 * g], acc0[4 * g + 1], acc0[4 * g + 2], acc0[4 * g + 3]};
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(f32x4 *)(ab + acc_off(px, 8 + 2 * g + hi)) =
                    f32x4{acc1[4 * g], acc1[4 * g + 1], acc1[4 * g + 2], acc1[4 * g + 3]};
            // publishes the results; the epilogue waves' rows for the next step land
            lds_barrier();
            cbuf ^= 1;
        }
        lds_barrier();   // the epilogue waves' last results
        __syncthreads();   // the statistics combination
        return;
    }

    // Epilogue waves: lane l holds channels 8 (l % 8) .. + 7 of pixels 8 r + l / 8 of its
    // 32-pixel quarter of a step.  Running statistics per lane: sums of deviations from a
    // shift (the lane's first value of each channel) and of their squares, and the count.
    const int ew = wave - NMW, c8 = lane & 7, et = tid - NMW * 64;
    float c[8], s1[8], s2[8], cnt = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        c[i] = 0.f;
        s1[i] = 0.f;
        s2[i] = 0.f;
    }
    bool first = true;   // wave-uniform
    // sc1 without nt: the z lines then still sit in the last-level cache for the
    // normalisation pass that reads them next.
    constexpr int Z_POLICY = 16;
    // Step (n_, a_, npix_)'s results in buffer buf: statistics, bf16 z to global memory.
    // Every row of the buffer holds a value of each channel (pixels past the step were
    // computed as the step's first pixel), so the shifts set from the first finished step
    // are valid.
    auto finish_t = [&](auto masked, int buf, int n_, int a_, int npix_) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked)::value;
        const uint8_t *ab = accb + buf * ACC_BYTES;
        const __amdgpu_buffer_rsrc_t zr = make_rsrc(p.z + ((size_t)n_ * PQ + a_) * HK, npix_ * HK * 2);
        float v[4][8];   // all eight reads in flight at once
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int px = 32 * ew + 8 * r + (lane >> 3);
            const f32x4 lo = *(const f32x4 *)(ab + acc_off(px, 2 * c8));
            const f32x4 hv = *(const f32x4 *)(ab + acc_off(px, 2 * c8 + 1));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[r][e] = lo[e];
                v[r][4 + e] = hv[e];
            }
        }
        if (first) {
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = v[0][i];
            first = false;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int px = 32 * ew + 8 * r + (lane >> 3);
            const u32x4 o = {pack_bf16x2(v[r][0], v[r][1]), pack_bf16x2(v[r][2], v[r][3]),
                             pack_bf16x2(v[r][4], v[r][5]), pack_bf16x2(v[r][6], v[r][7])};
            __builtin_amdgcn_raw_buffer_store_b128(o, zr, px * (HK * 2) + 16 * c8, 0, Z_POLICY);
            const bool use = !MASKED || px < npix_;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float d = v[r][i] - c[i];
                if constexpr (MASKED) d = use ? d : 0.f;
                s1[i] += d;
                s2[i] = fmaf(d, d, s2[i]);
            }
            if constexpr (MASKED) cnt += use ? 1.f : 0.f;
        }
        if constexpr (!MASKED) cnt += 4.f;
    };
    auto finish = [&](int buf, int n_, int a_, int npix_) __attribute__((always_inline)) {
        if (npix_ == WSP)
            finish_t(std::false_type{}, buf, n_, a_, npix_);
        else
            finish_t(std::true_type{}, buf, n_, a_, npix_);
    };

    // Row pieces travel two steps ahead: the rows step u adds are loaded into registers
    // during step u - 2 and widened into their slots during step u - 1 (slots no wave of
    // that step reads), so each load has a whole step to land.
    struct Pieces {
        Piece d[PPT];
        int la[PPT];   // LDS byte offset of the widened piece
        bool on[PPT];
    };
    // Piece k of this thread is, in every step, piece g of the ri-th row the step adds
    // (i = et + 256 k = ri * W / 8 + g): its offsets from the step's first row, in x and in
    // the ring, are fixed.
    int p_ri[PPT], p_xo[PPT], p_lo[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int i = et + NET * k;
        const int ri = div_m(i, p.mG);
        const int g = i - ri * gpr;
        p_ri[k] = ri;
        p_xo[k] = ri * (W * 6) + g * 48;
        p_lo[k] = ri * SB + (p.pw + 8 * g) * 8;
    }
    // The rows step u adds after the range's previous step, at most PPT pieces per thread:
    // in the same image (u.s > 0), input rows 2 olr(u.s - 1) - ph + R .. 2 olr(u.s) - ph +
    // R - 1; an image's first step, its rows -ph .. 2 olr(0) - ph + R - 1.
    // These loads are buffer loads in inline assembly (an offset past the end of x reads
    // zeros), outside the compiler's wait tracking: each step issues exactly 3 PPT of them,
    // and the widening of a set waits (vmcnt) for exactly the memory operations issued
    // after it.  Left to the compiler, every widening waited for all outstanding
    // operations, the loads just issued for the step after included.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, p.N * H * W * 3 * 2);
    auto buf_ld = [&](int off) {
        u32x4 v;
        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(off), "s"(xr) : "memory");
        return v;
    };
    auto load_rows = [&](Pieces &pc, const StepIt &u, bool exists) __attribute__((always_inline)) {
        int h0, v0, nrows;
        if (u.s > 0) {
            const int olrp = div_m(u.s * WSP - 1, p.mQ);
            const int au = u.s * WSP;
            const int olru = div_m(au + min(WSP, PQ - au) - 1, p.mQ);
            h0 = 2 * olrp - p.ph + R;
            nrows = 2 * (olru - olrp);
            v0 = u.img * VPI + 2 * olrp + R;
        } else {
            const int olr0 = div_m(min(WSP, PQ) - 1, p.mQ);
            h0 = -p.ph;
            nrows = 2 * olr0 + R;
            v0 = u.img * VPI;
        }
        if (!exists) nrows = 0;
        const int sl_0 = v0 % NSLOT;
        const int xrow0 = (u.n * H + h0) * (W * 6);   // byte offset of the step's first row
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int ri = p_ri[k], h = h0 + ri;
            pc.on[k] = ri < nrows;
            pc.la[k] = sl_0 * SB + p_lo[k] - (sl_0 + ri >= NSLOT ? NSLOT * SB : 0);
            const int off = pc.on[k] && h >= 0 && h < H ? xrow0 + p_xo[k] : (int)0x80000000u;
            pc.d[k].a = buf_ld(off);
            pc.d[k].b = buf_ld(off + 16);
            pc.d[k].d = buf_ld(off + 32);
        }
    };
    // Waits until at most N of this wave's memory operations are outstanding, then ties a
    // set's registers to the wait, so that no use of them is placed above it.
    auto vm_wait_set = [&](int n, Pieces &pc) {
        if (n >= 14) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
        else if (n >= 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
#pragma unroll
        for (int k = 0; k < PPT; ++k) asm volatile("" : "+v"(pc.d[k].a), "+v"(pc.d[k].b), "+v"(pc.d[k].d));
    };
    static_assert(PPT == 2, "the wait counts below assume 6 loads per step");
    auto advance = [&](StepIt &u) {
        if (++u.s == spi) {
            ++u.n;
            ++u.img;
            u.s = 0;
        }
    };

    int pn = 0, pa = 0, pnpix = 0, pbuf = 0;                 // the previous step (pnpix 0: none)
    int cbuf = 0;
    StepIt it = it0, it2 = it0;                               // steps t and t + 2
    advance(it2);
    Pieces pA, pB;   // the rows of steps t + 1 and t + 2, the two sets swapping roles each step
    load_rows(pA, it2, t0 + 1 < t1);
    advance(it2);
    // Step t: loads the rows of step t + 2 into `nxt` (6 loads), finishes step t - 1 (4
    // stores, from step t0 + 1 on), stores `cur` (the rows of step t + 1, loaded during
    // step t - 1, or before the loop for t = t0).  The operations issued after cur's loads
    // are then 6 at t0, 10 at t0 + 1 and 4 + 6 + 4 = 14 after.  The loop is unrolled by
    // two so that the sets swap roles without register copies (a copy would wait for the
    // loads it was meant to overlap).
    auto step = [&](int t, Pieces &cur, Pieces &nxt) __attribute__((always_inline)) {
        load_rows(nxt, it2, t + 2 < t1);
        if (pnpix > 0) finish(pbuf, pn, pa, pnpix);
        vm_wait_set(t >= t0 + 2 ? 14 : t == t0 + 1 ? 10 : 6, cur);
        // The next step's rows into their slots (no wave of this step reads them).
#pragma unroll
        for (int k = 0; k < PPT; ++k)
            if (cur.on[k]) store_piece_at(lds + cur.la[k], cur.d[k]);
        // The barrier publishes this step's results and the next step's rows, and frees
        // the result buffer read here for the next step's MFMAs.
        lds_barrier();
        pn = it.n;
        pa = it.s * WSP;
        pnpix = min(WSP, PQ - pa);
        pbuf = cbuf;
        cbuf ^= 1;
        advance(it);
        advance(it2);
    };
    for (int t = t0; t < t1; t += 2) {
        step(t, pA, pB);
        if (t + 1 < t1) step(t + 1, pB, pA);
    }
    // The last step's loads (of rows no step needs) are still in flight: they must land
    // before their registers are used for anything else.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        asm volatile("" : "+v"(pA.d[k].a), "+v"(pA.d[k].b), "+v"(pA.d[k].d));
        asm volatile("" : "+v"(pB.d[k].a), "+v"(pB.d[k].b), "+v"(pB.d[k].d));
    }
    if (pnpix > 0) finish(pbuf, pn, pa, pnpix);
    lds_barrier();   // every wave is done with the result buffers and the ring

    // Statistics: each lane's (count n, mean = c + s1/n, M2 = s2 - s1^2/n), combined by the
    // law of total variance (mean = sum n_l mean_l / n, M2 = sum [M2_l + n_l (mean_l -
    // mean)^2]) over the 8 lanes that hold the same channels (lane shuffles, fp32; both
    // operands of every addition are the same at every lane of the group, so the sums are
    // identical across it), then over the 4 epilogue waves in fp64, one thread per channel:
    // row blockIdx.x of the partials (means then M2 of the 64 channels; the count at
    // partials[gridDim.x * 128 + blockIdx.x]).
    float *st = (float *)lds;                                 // [NEW][8][17]
    {
        const float rc = cnt > 0.f ? 1.f / cnt : 0.f;
        float ml[8], qv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ml[i] = c[i] + s1[i] * rc;
            qv[i] = fmaxf(s2[i] - s1[i] * s1[i] * rc, 0.f);
        }
        auto gsum = [](float v) {
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            return v;
        };
        const float nr = gsum(cnt);
        const float rn = nr > 0.f ? 1.f / nr : 0.f;
        float mr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) mr[i] = gsum(cnt * ml[i]) * rn;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float d = ml[i] - mr[i];
            qv[i] = gsum(fmaf(cnt * d, d, qv[i]));
        }
        if (lane < 8) {
            float *e = st + (ew * 8 + lane) * 17;
            e[0] = nr;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[1 + i] = mr[i];
                e[9 + i] = qv[i];
            }
        }
    }
    __syncthreads();
    if (et < HK) {
        const int k = et, g8 = k >> 3, i = k & 7;
        double nsum = 0.0, sm = 0.0;
#pragma unroll
        for (int w = 0; w < NEW; ++w) {
            const float *en = st + (w * 8 + g8) * 17;
            nsum += (double)en[0];
            sm += (double)en[0] * (double)en[1 + i];
        }
        const double mean = nsum > 0.0 ? sm / nsum : 0.0;
        double m2 = 0.0;
#pragma unroll
        for (int w = 0; w < NEW; ++w) {
            const float *en = st + (w * 8 + g8) * 17;
            const double d = (double)en[1 + i] - mean;
            m2 += (double)en[9 + i] + (double)en[0] * d * d;
        }
        float *out = p.partials + (size_t)blockIdx.x * 2 * HK;
        out[k] = (float)mean;
        out[HK + k] = (float)m2;
        if (k == 0) p.partials[(size_t)gridDim.x * 2 * HK + blockIdx.x] = (float)nsum;
    }
}

// Widened pixels per staged row: up to the last one a read reaches (2 (Q - 1) + 7) and
// past the image's right edge, rounded up to even so that slots start on 16 bytes.
int c3p_lw(const ConvGeom &g)
{
    const int lw = std::max(2 * (g.Q - 1) + 8, g.pw + g.W);
    return lw + (lw & 1);
}

// Ring slots and row pieces per step.  While step s computes, the ring holds the rows it
// reads and the rows the range's next step adds: in the same image, virtual rows 2 ofr(s)
// .. 2 olr(s + 1) + R - 1; at an image's last step, 2 ofr(s) .. VPI - 1 of this image and
// 0 .. 2 olr(0) + R - 1 of the next.  Exact over the steps of one image (every image has
// the same steps).
struct C3Ring {
    int nslot;        // slots
    int pieces;       // 8-pixel pieces one step adds, at most
};
C3Ring c3p_ring(const ConvGeom &g)
{
    const int PQ = g.P * g.Q, spi = (PQ + WSP - 1) / WSP, gpr = g.W / 8, vpi = 2 * (g.P - 1) + g.R;
    const int olr0 = (std::min(WSP, PQ) - 1) / g.Q;
    C3Ring r{2 * olr0 + g.R, 0};
    for (int s = 0; s < spi; ++s) {
        const int a = s * WSP, npix = std::min(WSP, PQ - a);
        const int ofr = a / g.Q, olr = (a + npix - 1) / g.Q;
        int need, rows;
        if (s + 1 < spi) {
            const int a1 = a + WSP;
            const int olr1 = (a1 + std::min(WSP, PQ - a1) - 1) / g.Q;
            need = 2 * (olr1 - ofr) + g.R;
            rows = 2 * (olr1 - olr);
        } else {
            need = vpi - 2 * ofr + 2 * olr0 + g.R;
            rows = 2 * olr0 + g.R;
        }
        r.nslot = std::max(r.nslot, need);
        r.pieces = std::max(r.pieces, rows * gpr);
    }
    return r;
}

template <int R>
hipError_t launch_c3p(const C3PParams &prm, const ConvGeom &g, size_t lds, hipStream_t st, hipEvent_t e0,
                      hipEvent_t e1)
{
    const hipError_t e = raise_lds_limit((const void *)conv_c3s2_ws_kernel<R>, (int)lds);
    if (e != hipSuccess) return e;
    return launch(conv_c3s2_ws_kernel<R>, dim3(c3s2_grid(g)), dim3(NT), (uint32_t)lds, st, e0, e1, prm);
}

}  // namespace

bool c3s2_eligible(const ConvGeom &g)
{
    if (!(g.C == 3 && g.K == HK && g.sh == 2 && g.sw == 2 && g.R >= 1 && g.R <= MAXR && g.S >= 1 && g.S <= 8 &&
          g.W % 8 == 0 && g.ph >= 0 && g.pw >= 0 && g.P >= 1 && g.Q >= 1))
        return false;
    // zero columns left and right of the image: at most 16 per row
    if (c3p_lw(g) - g.W > 16 || c3p_lw(g) < g.pw + g.W) return false;
    // the multiply-high divisions: pixel indices below 2^32 / Q
    if ((uint64_t)((size_t)g.P * g.Q + WSP) * g.Q >= (1ull << 32)) return false;
    if ((size_t)g.N * g.P * g.Q * HK * 2 >= 0x7fffffffu || (size_t)g.N * g.H * g.W * 3 * 2 >= 0x7fffffffu ||
        (size_t)g.N * (2 * (g.P - 1) + g.R) >= 0x7fffffffu)
        return false;
    // at most PPT pieces per epilogue thread of the rows a step adds
    if (c3p_ring(g).pieces > PPT * NET) return false;
    return c3s2_lds_bytes(g) <= 160 * 1024;
}

int c3s2_grid(const ConvGeom &g)
{
    const long steps = (long)g.N * ((g.P * g.Q + WSP - 1) / WSP);
    return (int)std::min<long>(steps, 256);
}

size_t c3s2_lds_bytes(const ConvGeom &g)
{
    return std::max((size_t)c3p_ring(g).nslot * c3p_lw(g) * 8 + 2 * ACC_BYTES, (size_t)EST_BYTES);
}

hipError_t launch_conv_c3s2_stats(const ConvGeom &g, const uint16_t *x, const uint16_t *w, uint16_t *z,
                                  float *partials, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    static_assert(HK * MAXR * 32 * 2 <= ACC_BYTES, "the widened filter fits one result buffer");
    C3PParams prm;
    prm.x = x;
    prm.w = w;
    prm.z = z;
    prm.partials = partials;
    prm.N = g.N;
    prm.H = g.H;
    prm.W = g.W;
    prm.R = g.R;
    prm.S = g.S;
    prm.ph = g.ph;
    prm.pw = g.pw;
    prm.P = g.P;
    prm.Q = g.Q;
    prm.slot_bytes = c3p_lw(g) * 8;
    prm.nslot = c3p_ring(g).nslot;
    prm.vpi = 2 * (g.P - 1) + g.R;
    prm.mQ = (uint32_t)(((1ull << 32) + g.Q - 1) / g.Q);                 // 0 for Q = 1
    prm.mG = (uint32_t)(((1ull << 32) + g.W / 8 - 1) / (g.W / 8));       // 0 for W = 8
    const size_t lds = c3s2_lds_bytes(g);
    switch (g.R) {
    case 1: return launch_c3p<1>(prm, g, lds, st, e0, e1);
    case 2: return launch_c3p<2>(prm, g, lds, st, e0, e1);
    case 3: return launch_c3p<3>(prm, g, lds, st, e0, e1);
    case 4: return launch_c3p<4>(prm, g, lds, st, e0, e1);
    case 5: return launch_c3p<5>(prm, g, lds, st, e0, e1);
    case 6: return launch_c3p<6>(prm, g, lds, st, e0, e1);
    case 7: return launch_c3p<7>(prm, g, lds, st, e0, e1);
    default: return hipErrorInvalidValue;   // not eligible
    }
}

}  // namespace cbr
