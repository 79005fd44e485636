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
// The schedule is that of the persistent 3x3 kernel (conv3x3_c64.hip):
//   - One 512-thread workgroup per CU walks a contiguous range of the batch's steps of
//     SP = 256 output pixels (8 blocks of 32, NHWC order, starting anywhere in a row);
//     SIMD s takes blocks s and s + 4, the two waves of a SIMD the two channel halves.
//   - Wave w keeps its half of the widened filter in registers (2R fragments).
//   - LDS holds a ring of widened input rows: row h (-ph <= h) in slot (h + ph) % nslot,
//     zero columns on both sides; rows outside the image are zero rows.  While a step
//     computes, each thread holds one 8-pixel piece of the rows the next step adds (three
//     16-byte loads issued at the step's start); after the step's k-loops it widens the
//     piece into its slot, which no wave of the step reads.
//   - z goes through two LDS staging buffers and leaves, during the next step, as 1 KB
//     runs of whole 128-byte pixel rows; the statistics are kept per lane as shifted sums
//     and combined once at the end into one (count, mean, M2) row per workgroup.
#include "cbr_launch.h"
#include "cbr_persist.h"

namespace cbr {
namespace {

using namespace persist;

constexpr int MAXR = 7;    // filter rows

struct C3PParams {
    const uint16_t *x;      // N x H x W x 3
    const uint16_t *wexp;   // 64 x R x 8 x 4 (zero-padded filter)
    uint16_t *z;            // N x P x Q x 64
    float *partials;        // [gridDim.x][2][64] means and M2, then [gridDim.x] counts
    int N, H, W, R, ph, pw, P, Q;
    int slot_bytes;         // LW * 8: widened pixels per staged row, zero columns included
    int nslot;              // ring slots
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

// Widened filter [64][R][8][4] <- KRSC [64][R][S][3], zeros elsewhere.
__global__ __launch_bounds__(256) void widen_filter_c3_kernel(const uint16_t *__restrict__ w, int R, int S,
                                                             uint16_t *__restrict__ wexp)
{
    const int total = HK * R * 32;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
        const int c = i & 3, s = (i >> 2) & 7, kr = i >> 5;          // kr = k*R + r
        wexp[i] = (c < 3 && s < S) ? w[((size_t)kr * S + s) * 3 + c] : (uint16_t)0;
    }
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

// R (the filter's rows) is a template parameter: the k-loops are then straight-line code
// (2R fragment reads, then 2R MFMAs), with no run-time guards between the reads.
template <int R>
__global__ __launch_bounds__(NT, 1) void conv_c3s2_persist_kernel(C3PParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int simd = wave & (NSIMD - 1), j = wave >> 2;
    const int hi = lane >> 5, l32 = lane & 31;
    const int H = p.H, W = p.W, Q = p.Q, SB = p.slot_bytes, NSLOT = p.nslot;
    const int PQ = p.P * Q;
    const int spi = (PQ + SP - 1) / SP;                       // steps per image
    // This workgroup's steps: a contiguous range [t0, t1) of the N * spi steps of the batch
    // (step s of image n is step n * spi + s), spread evenly over the grid.
    const long tot = (long)p.N * spi;
    const int t0 = (int)(tot * blockIdx.x / gridDim.x), t1 = (int)(tot * (blockIdx.x + 1) / gridDim.x);
    const int gpr = W / 8;                                    // 8-pixel pieces per input row
    constexpr int nks = 2 * R;
    uint8_t *const stg0 = lds + NSLOT * SB;                   // two z staging buffers

    // Filter fragment t (k-step t): lane (l32, hi) holds output channel 32j + l32, tap row
    // t / 2, taps 4 (t % 2) + 2 hi and + 1, four channels each: 16 bytes of wexp.
    bf16x8 wf[nks];
#pragma unroll
    for (int t = 0; t < nks; ++t)
        wf[t] = *(const bf16x8 *)(p.wexp + ((size_t)(32 * j + l32) * R + (t >> 1)) * 32 + 16 * (t & 1) + 8 * hi);

    // Piece g of input row h of image n (zeros outside the image), and its widened store
    // into the row's slot: pixel u of the row at byte (pw + u) * 8 of the slot.
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
    auto store_piece = [&](int h, int g, const Piece &r) {
        uint8_t *dst = lds + ((h + p.ph) % NSLOT) * SB + (p.pw + 8 * g) * 8;
        const uint32_t v[12] = {r.a[0], r.a[1], r.a[2], r.a[3], r.b[0], r.b[1], r.b[2], r.b[3], r.d[0], r.d[1], r.d[2], r.d[3]};
        // bf16 value t of the piece is half t % 2 of word t / 2; pixel e is values 3e .. 3e + 2
        auto half = [&](int t) { return (v[t >> 1] >> (16 * (t & 1))) & 0xffffu; };
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *(u32x2 *)(dst + e * 8) = u32x2{half(3 * e) | (half(3 * e + 1) << 16), half(3 * e + 2)};
    };
    // Rows h0 .. h0 + nrows - 1 of image n, every piece, loaded and stored in place.
    auto stage_rows = [&](int n, int h0, int nrows) {
        for (int i = tid; i < nrows * gpr; i += NT) {
            const int ri = div_m(i, p.mG);
            const int g = i - ri * gpr;
            store_piece(h0 + ri, g, load_piece(n, h0 + ri, g));
        }
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
    int n = t0 / spi, s = t0 - n * spi;                      // image and step of step t
    if (t1 > t0) {
        // the first step's input rows 2 ofr - ph .. 2 olr - ph + R - 1
        const int a = s * SP, npix = min(SP, PQ - a);
        const int ofr = div_m(a, p.mQ), olr = div_m(a + npix - 1, p.mQ);
        stage_rows(n, 2 * ofr - p.ph, 2 * (olr - ofr) + R);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    float c[8], s1[8], s2[8], cnt = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        c[i] = 0.f;
        s1[i] = 0.f;
        s2[i] = 0.f;
    }
    bool first = true;   // wave-uniform: the wave's first pixel block sets the shifts
    Staged prev;         // the previous step, staged in buffer pbuf
    prev.nq = 0;
    prev.zr = make_rsrc(p.z, 0);   // nothing staged yet: every store is dropped
    int pbuf = 1;
    // sc1 without nt: the z lines then still sit in the last-level cache for the
    // normalisation pass that reads them next.
    constexpr int Z_POLICY = 16;

    for (int t = t0; t < t1; ++t, ++s) {
        if (s == spi) {
            // The next image: every wave is past the last step's reads; stage the rows of
            // its first step.
            ++n;
            s = 0;
            const int olr0 = div_m(min(SP, PQ) - 1, p.mQ);
            stage_rows(n, -p.ph, 2 * olr0 + R);
            lds_barrier();
        }
        const int a = s * SP;                                   // first pixel of the step
        const int npix = min(SP, PQ - a);
        const int nblk = (npix + 31) >> 5;
        const int nb = (simd < nblk) + (simd + NSIMD < nblk);
        const bool full = npix == 32 * nblk;
        const int ofr = div_m(a, p.mQ), olr = div_m(a + npix - 1, p.mQ);
        // The rows the next step of the range adds (none at an image's or the range's end):
        // input rows 2 olr - ph + R .. 2 olr1 - ph + R - 1, at most one piece per thread.
        Piece nx;
        int nx_h = 0, nx_g = 0;
        bool nx_on = false;
        if (t + 1 < t1 && s + 1 < spi) {
            const int a1 = a + SP;
            const int olr1 = div_m(a1 + min(SP, PQ - a1) - 1, p.mQ);
            if (tid < 2 * (olr1 - olr) * gpr) {
                const int ri = div_m(tid, p.mG);
                nx_g = tid - ri * gpr;
                nx_h = 2 * olr - p.ph + R + ri;
                nx = load_piece(n, nx_h, nx_g);
                nx_on = true;
            }
        }
        // The previous step's z: channel half 0's waves store the first half of its runs,
        // the others the second half.  Half 0 stores at the step's start and half 1 after
        // its first block, so the two waves of a SIMD leave the barrier out of phase: one's
        // k-loop runs beside the other's stores or epilogue instead of both competing for
        // the MFMA unit and then both leaving it idle.
        auto store_prev = [&]() {
            if (prev.nq > 0) {
                const uint8_t *sb = stg0 + pbuf * STG_BYTES;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int q = simd + NSIMD * (4 * j + k);
                    const int px = 8 * q + (lane >> 3);
                    prev.d[k] = *(const u32x4 *)(sb + px * PXB + (((lane & 7) ^ perm(px)) << 4));
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int q = simd + NSIMD * (4 * j + k);
                    __builtin_amdgcn_raw_buffer_store_b128(prev.d[k], prev.zr, q * 1024 + lane * 16, 0, Z_POLICY);
                }
            }
        };
        if (j == 0 || nb == 0) store_prev();
        const int cbuf = pbuf ^ 1;
        uint8_t *const stg = stg0 + cbuf * STG_BYTES;
        // slot of input row 2 ofr - ph (tap row 0 of the step's first output row)
        const int fslot = (2 * ofr) % NSLOT;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            if (bb >= nb) break;
            const int px = 32 * (simd + NSIMD * bb) + l32;      // pixel within the step
            const bool use = px < npix;
            const int pi = a + (use ? px : 0);
            const int pr = div_m(pi, p.mQ);
            const int q = pi - pr * Q;
            // tap row r of output row pr reads input row 2 pr - ph + r, in slot
            // (2 pr + r) % nslot
            int sl0 = fslot + 2 * (pr - ofr);
            while (sl0 >= NSLOT) sl0 -= NSLOT;
            const int colb = 16 * q + 16 * hi;
            const uint32_t lbase = (uint32_t)(uintptr_t)(lds_u8 *)lds + colb;
            bf16x8 xf[nks];
#pragma unroll
            for (int tt = 0; tt < nks; ++tt) {
                int sl = sl0 + (tt >> 1);
                if (sl >= NSLOT) sl -= NSLOT;
                xf[tt] = lds_rd(lbase + sl * SB + 32 * (tt & 1));
            }
            f32x16 acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.f;
            mfma_chain<R, 0>(acc, wf, xf);
            if (full)
                epilogue<false>(acc, use, true, first, stg, px, j, hi, c, s1, s2, cnt);
            else
                epilogue<true>(acc, use, (px ^ 16) < npix, first, stg, px, j, hi, c, s1, s2, cnt);
            first = false;
            if (bb == 0 && j == 1) store_prev();
        }
        // The next step's rows into their slots (no wave of this step reads them).
        if (nx_on) store_piece(nx_h, nx_g, nx);
        // The barrier publishes the staged rows and this step's staged z, and frees the
        // staging buffer the previous step's z was read from; the z stores run on.
        lds_barrier();
        prev.nq = (npix + 7) / 8;
        prev.zr = make_rsrc(p.z + ((size_t)n * PQ + a) * HK, npix * HK * 2);
        pbuf = cbuf;
    }
    if (prev.nq > 0) {
        const uint8_t *sb = stg0 + pbuf * STG_BYTES;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int q = simd + NSIMD * (4 * j + k);
            const int px = 8 * q + (lane >> 3);
            prev.d[k] = *(const u32x4 *)(sb + px * PXB + (((lane & 7) ^ perm(px)) << 4));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int q = simd + NSIMD * (4 * j + k);
            __builtin_amdgcn_raw_buffer_store_b128(prev.d[k], prev.zr, q * 1024 + lane * 16, 0, Z_POLICY);
        }
    }
    lds_barrier();   // every wave is done with the staging buffers and the ring
    store_stat_row(lds, c, s1, s2, cnt, p.partials, blockIdx.x, gridDim.x);
}

// Widened pixels per staged row: up to the last one a read reaches (2 (Q - 1) + 7) and
// past the image's right edge, rounded up to even so that slots start on 16 bytes.
int c3p_lw(const ConvGeom &g)
{
    const int lw = std::max(2 * (g.Q - 1) + 8, g.pw + g.W);
    return lw + (lw & 1);
}
// Ring slots: the input rows of a step and the rows the next adds, 2 (olr(s + 1) - ofr(s))
// + R, where the output rows of 2 SP consecutive pixels span at most (2 SP - 1) / Q + 2.
int c3p_nslot(const ConvGeom &g) { return 2 * ((2 * SP - 1) / g.Q + 1) + g.R; }

template <int R>
hipError_t launch_c3p(const C3PParams &prm, const ConvGeom &g, size_t lds, hipStream_t st, hipEvent_t e1)
{
    const hipError_t e = raise_lds_limit((const void *)conv_c3s2_persist_kernel<R>, (int)lds);
    if (e != hipSuccess) return e;
    return launch(conv_c3s2_persist_kernel<R>, dim3(c3s2_grid(g)), dim3(NT), (uint32_t)lds, st, nullptr, e1, prm);
}

}  // namespace

bool c3s2_eligible(const ConvGeom &g)
{
    if (!(g.C == 3 && g.K == HK && g.sh == 2 && g.sw == 2 && g.R >= 1 && g.R <= MAXR && g.S >= 1 && g.S <= 8 &&
          g.W % 8 == 0 && g.ph >= 0 && g.pw >= 0 && g.P >= 1 && g.Q >= 1))
        return false;
    // zero columns left and right of the image: at most 16 per row
    if (c3p_lw(g) - g.W > 16 || c3p_lw(g) < g.pw + g.W) return false;
    // one piece per thread of the rows a step adds: 2 (SP / Q + 1) rows of W / 8 pieces
    if (2 * (SP / g.Q + 1) * (g.W / 8) > NT) return false;
    // the multiply-high divisions: pixel indices below 2^32 / Q
    if ((uint64_t)((size_t)g.P * g.Q + SP) * g.Q >= (1ull << 32)) return false;
    return c3s2_lds_bytes(g) <= 160 * 1024 && (size_t)g.N * g.P * g.Q * HK * 2 < 0x7fffffffu &&
           (size_t)g.N * g.H * g.W * 3 * 2 < 0x7fffffffu;
}

int c3s2_grid(const ConvGeom &g)
{
    const long steps = (long)g.N * ((g.P * g.Q + SP - 1) / SP);
    return (int)std::min<long>(steps, 256);
}

size_t c3s2_lds_bytes(const ConvGeom &g)
{
    return std::max((size_t)c3p_nslot(g) * c3p_lw(g) * 8 + 2 * STG_BYTES, (size_t)STATS_BYTES);
}

size_t c3s2_wexp_bytes(const ConvGeom &g) { return (size_t)HK * g.R * 32 * 2; }

hipError_t launch_conv_c3s2_stats(const ConvGeom &g, const uint16_t *x, const uint16_t *w, uint16_t *wexp,
                                  uint16_t *z, float *partials, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    hipError_t e = launch(widen_filter_c3_kernel, dim3((HK * g.R * 32 + 255) / 256), dim3(256), 0, st, e0, nullptr, w,
                          g.R, g.S, wexp);
    if (e != hipSuccess) return e;
    C3PParams prm;
    prm.x = x;
    prm.wexp = wexp;
    prm.z = z;
    prm.partials = partials;
    prm.N = g.N;
    prm.H = g.H;
    prm.W = g.W;
    prm.R = g.R;
    prm.ph = g.ph;
    prm.pw = g.pw;
    prm.P = g.P;
    prm.Q = g.Q;
    prm.slot_bytes = c3p_lw(g) * 8;
    prm.nslot = c3p_nslot(g);
    prm.mQ = (uint32_t)(((1ull << 32) + g.Q - 1) / g.Q);                 // 0 for Q = 1
    prm.mG = (uint32_t)(((1ull << 32) + g.W / 8 - 1) / (g.W / 8));       // 0 for W = 8
    const size_t lds = c3s2_lds_bytes(g);
    switch (g.R) {
    case 1: return launch_c3p<1>(prm, g, lds, st, e1);
    case 2: return launch_c3p<2>(prm, g, lds, st, e1);
    case 3: return launch_c3p<3>(prm, g, lds, st, e1);
    case 4: return launch_c3p<4>(prm, g, lds, st, e1);
    case 5: return launch_c3p<5>(prm, g, lds, st, e1);
    case 6: return launch_c3p<6>(prm, g, lds, st, e1);
    case 7: return launch_c3p<7>(prm, g, lds, st, e1);
    default: return hipErrorInvalidValue;   // not eligible
    }
}

}  // namespace cbr
