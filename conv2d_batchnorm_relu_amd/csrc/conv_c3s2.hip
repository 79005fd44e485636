// conv_c3s2.hip -- first-layer convolution (3 input channels, stride 2, up to 7x8
// taps, 64 output channels) fused with the per-channel sum and sum of squares of its
// output: the training forward's conv + genstats step (CBR page, section 4.1) for the
// network's input layer (the CBR page's first-layer special case, section 5.3, is the
// backward's skipped data gradient; this is its forward).
//
// With 3 channels a pixel is 6 bytes, so the generic implicit GEMM gathers element by
// element.  Here each workgroup owns TP = 4 output rows of one image.  It stages the
// 2*(TP-1) + R input rows it needs in LDS with every pixel widened to 4 channels (8
// bytes, the fourth zero) and zero columns on both sides, and the filter widened to
// [64][R][8][4] (taps s >= S and channel 3 zero).  The reduction is then ordered
// (r, s, c) with s and c innermost: for a fixed tap row r, the 16 values of one MFMA
// k-step are four consecutive input pixels x 4 channels, and because the stride is 2,
// the 8 values a lane needs for output column q are one aligned 16-byte LDS read at
// pixel 2q + s0.  Consecutive output columns read consecutive 16-byte chunks, so the
// reads are conflict-free.
//
// GEMM mapping: v_mfma_f32_32x32x16_bf16, filter as A (32 output channels), pixels as
// B (32 output pixels), 2*R k-steps (R*32 reduction values, S*3 of every 32 live).
// Four waves: wave w owns channel block w/2 and pixel blocks 7*(w%2) .. 7*(w%2)+6 of the
// band's 14 (4 rows x 112 columns for the 224x224 stem).  Two workgroups share a CU,
// so one's staging overlaps the other's MFMAs.
#include "cbr_launch.h"

namespace cbr {
namespace {

constexpr int NT = 256;
constexpr int TP = 4;          // output rows per workgroup
constexpr int KOUT = 64;       // output channels
constexpr int UPW = 7;         // pixel blocks per wave
constexpr int NBLK = 2 * UPW;  // pixel blocks per band (TP * Q <= 32 * NBLK)

struct C3Params {
    const uint16_t *x;      // N x H x W x 3
    const uint16_t *wexp;   // 64 x R x 8 x 4 (zero-padded filter)
    uint16_t *z;            // N x P x Q x 64
    float *partials;        // [gridDim.x][2][64] means and M2, then [gridDim.x] counts
    int N, H, W, R, ph, pw, P, Q;
    int bands;              // ceil(P / TP)
    int LW;                 // staged pixels per input row (zero columns included)
    int RB;                 // bytes per staged input row
    int WRB;                // bytes per staged filter row
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Chunk permutation of the z staging rows: 16-byte chunk c of pixel px sits at position
// c ^ perm(px), so consecutive pixels' chunks spread over the LDS banks.
__device__ __forceinline__ int perm(int px) { return (px >> 1) & 7; }

// Widened filter [64][R][8][4] <- KRSC [64][R][S][3], zeros elsewhere.
__global__ __launch_bounds__(NT) void widen_filter_c3_kernel(const uint16_t *__restrict__ w, int R, int S,
                                                             uint16_t *__restrict__ wexp)
{
    const int total = KOUT * R * 32;
    for (int i = blockIdx.x * NT + threadIdx.x; i < total; i += gridDim.x * NT) {
        const int c = i & 3, s = (i >> 2) & 7, kr = i >> 5;          // kr = k*R + r
        wexp[i] = (c < 3 && s < S) ? w[((size_t)kr * S + s) * 3 + c] : (uint16_t)0;
    }
}

__global__ __launch_bounds__(NT, 2) void conv_c3s2_stats_kernel(C3Params p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int NR = 2 * (TP - 1) + p.R;              // staged input rows
    uint8_t *wl = lds;                              // KOUT x WRB
    uint8_t *xl = lds + KOUT * p.WRB;               // NR x RB
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = blockIdx.x / p.bands, band = blockIdx.x - n * p.bands;
    const int p0 = band * TP;
    const int h0 = 2 * p0 - p.ph;                   // input row of staged row 0
    const int W = p.W, Q = p.Q;

    // The staging loops index with lane bit fields, not divisions: an integer division
    // by a run-time value is some forty vector instructions.
    // Filter: R*4 <= 32 16-byte chunks per output channel; lane bits 0..4 pick the chunk.
    {
        const int cpr = p.R * 4, ch = tid & 31;
        if (ch < cpr)
            for (int k = tid >> 5; k < KOUT; k += NT / 32)
                *(u32x4 *)(wl + k * p.WRB + ch * 16) = ((const u32x4 *)p.wexp)[k * cpr + ch];
    }
    // Input rows.  Zero: rows outside the image, and the columns left and right of the
    // image (staged pixel j holds input column j - pw; at most 16 of them per row).  Image
    // pixels: groups of 8 (48 bytes = three 16-byte loads), widened to 8 bytes each.
    const int gpr = W / 8;                          // pixel groups per row
    const int npad = p.LW - W;                      // zero columns per row, <= 16
    for (int i = tid >> 4; i < NR; i += NT / 16) {
        const int h = h0 + i, c = tid & 15;
        if (h >= 0 && h < p.H) {
            if (c < npad) {
                const int j = c < p.pw ? c : W + c;
                *(u32x2 *)(xl + i * p.RB + j * 8) = u32x2{0u, 0u};
            }
        } else {
            for (int j = c; j < p.LW; j += 16) *(u32x2 *)(xl + i * p.RB + j * 8) = u32x2{0u, 0u};
        }
    }
    for (int i = tid >> 5; i < NR; i += NT / 32) {
        const int h = h0 + i;
        if (h < 0 || h >= p.H) continue;
        for (int gi = tid & 31; gi < gpr; gi += 32) {
        const u32x4 *src = (const u32x4 *)(p.x + (((size_t)n * p.H + h) * W + 8 * gi) * 3);
        const u32x4 a = src[0], b = src[1], d = src[2];
        const uint32_t v[12] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3], d[0], d[1], d[2], d[3]};
        uint8_t *dst = xl + i * p.RB + (p.pw + 8 * gi) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // bf16 values 3e, 3e+1, 3e+2 of the group; value t is half t%2 of word t/2.
            auto half = [&](int t) { return (v[t >> 1] >> (16 * (t & 1))) & 0xffffu; };
            const uint32_t lo = half(3 * e) | (half(3 * e + 1) << 16);
            *(u32x2 *)(dst + e * 8) = u32x2{lo, half(3 * e + 2)};
        }
        }
    }
    __syncthreads();

    // Wave's channel block and pixel blocks; per-block staged-pixel base of its lane.
    const int j = wave >> 1, blk0 = UPW * (wave & 1);
    const int hi = lane >> 5, l32 = lane & 31;
    const int wa = (32 * j + l32) * p.WRB + hi * 16;
    int xa[UPW];
    bool valid[UPW];
    const float invQ = 1.0f / (float)Q;
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
        const int pi = 32 * (blk0 + u) + l32;           // pixel within the band
        int pr = (int)((float)pi * invQ);               // pi / Q, corrected below
        pr -= pr * Q > pi;
        pr += (pr + 1) * Q <= pi;
        const int q = pi - pr * Q;
        valid[u] = pr < TP && p0 + pr < p.P;
        xa[u] = valid[u] ? KOUT * p.WRB + 2 * pr * p.RB + 2 * q * 8 + hi * 16 : KOUT * p.WRB;
    }

    // k-step t: tap row r = t/2, taps s = 4*(t%2) .. +3 (lane half hi: two of them).
    const int nks = 2 * p.R;
    f32x16 acc[UPW];
#pragma unroll
    for (int u = 0; u < UPW; ++u)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[u][v] = 0.f;
    bf16x8 af[2], bf[2][UPW];
    auto rd = [&](int t, int b) {
        const int r = t >> 1, hf = t & 1;
        af[b] = *(const bf16x8 *)(lds + wa + r * 64 + hf * 32);
#pragma unroll
        for (int u = 0; u < UPW; ++u) bf[b][u] = *(const bf16x8 *)(lds + xa[u] + r * p.RB + hf * 32);
    };
    rd(0, 0);
    for (int t = 0; t < nks; t += 2) {
        rd(t + 1, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < UPW; ++u)
            acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bf[0][u], acc[u], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (t + 2 < nks) rd(t + 2, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < UPW; ++u)
            acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], bf[1][u], acc[u], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }

    // Epilogue: lane holds, for pixel l32 of each block, channels 32j + 8g + 4hi + e in
    // acc[u][4g + e].  Per-lane statistics; z goes through LDS (the staged rows and the
    // filter are free once every wave is past the barrier) into pixel-major order, 16-byte
    // chunk c of band pixel px at (c ^ perm(px)) << 4, and leaves as 1 KB runs of whole
    // 128-byte pixel rows: storing straight from the MFMA layout touches 32 cache lines per
    // instruction with 16 bytes each, which the memory pipeline processes line by line.
    // Statistics, first pass: per-lane channel sums over the valid pixels.
    float s1[4][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) s1[g][e] = 0.f;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
        if (!valid[u]) continue;
        const int px = 32 * (blk0 + u) + l32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float a0 = acc[u][4 * g], a1 = acc[u][4 * g + 1];
            const float a2 = acc[u][4 * g + 2], a3 = acc[u][4 * g + 3];
            *(u32x2 *)(lds + px * 128 + (((4 * j + g) ^ perm(px)) << 4) + 8 * hi) =
                u32x2{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
            s1[g][0] += a0;
            s1[g][1] += a1;
            s1[g][2] += a2;
            s1[g][3] += a3;
        }
    }
    __syncthreads();
    // The band's rows are contiguous in z (NHWC): npx pixels from pixel (n, p0, 0).
    const int npx = min(TP, p.P - p0) * Q;
    {
        const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
            p.z + ((size_t)n * p.P + p0) * Q * KOUT, 0, npx * KOUT * 2, 0x00020000);
        // sc1 without nt: measured, the z lines then still sit in the last-level cache for
        // the normalisation pass that reads them next, and the stores run as fast.
        constexpr int Z_POLICY = 16;
        for (int q = wave; q < (npx + 7) / 8; q += NT / 64) {
            const int px = 8 * q + (lane >> 3);   // runs past npx: the buffer drops the store
            const u32x4 v = *(const u32x4 *)(lds + px * 128 + (((lane & 7) ^ perm(px)) << 4));
            __builtin_amdgcn_raw_buffer_store_b128(v, zr, q * 1024 + lane * 16, 0, Z_POLICY);
        }
    }

    // Cross-lane reductions through LDS, once every wave has read its z runs:
    // st[f][tid], f = 4*g + e for channel 32j + 8g + 4hi + e.  Thread (f, jj, h) of the
    // first 128 sums the 64 lanes of channel block jj with hi == h (waves 2jj and 2jj + 1
    // x 32 lanes) in a fixed order.
    __syncthreads();
    float *st = (float *)lds;            // 16 x NT floats = 16 KB
    float *bmean = st + 16 * NT;         // the band's 64 channel means
    auto reduce = [&](int f, int jj, int h) {
        float a = 0.f;
#pragma unroll
        for (int w = 2 * jj; w < 2 * jj + 2; ++w) {
            const f32x4 *row = (const f32x4 *)(st + f * NT + 64 * w + 32 * h);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4 q = row[i];
                a += (q[0] + q[1]) + (q[2] + q[3]);
            }
        }
        return a;
    };
    const int rf = tid >> 2, rjj = (tid >> 1) & 1, rh = tid & 1;      // reducing thread's role
    const int rk = 32 * rjj + 8 * (rf >> 2) + 4 * rh + (rf & 3);      // its channel
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[(4 * g + e) * NT + tid] = s1[g][e];
    __syncthreads();
    if (tid < 64) bmean[rk] = reduce(rf, rjj, rh) / (float)npx;
    __syncthreads();
    // Second pass: squared deviations of the valid pixels from the band's means.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const f32x4 m4 = *(const f32x4 *)(bmean + 32 * j + 8 * g + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s2 = 0.f;
#pragma unroll
            for (int u = 0; u < UPW; ++u) {
                const float d = acc[u][4 * g + e] - m4[e];
                s2 = valid[u] ? fmaf(d, d, s2) : s2;
            }
            st[(4 * g + e) * NT + tid] = s2;
        }
    }
    __syncthreads();
    if (tid < 64) {
        float *row = p.partials + (size_t)blockIdx.x * 2 * KOUT;
        row[rk] = bmean[rk];
        row[KOUT + rk] = reduce(rf, rjj, rh);
    }
    if (tid == 0) p.partials[(size_t)gridDim.x * 2 * KOUT + blockIdx.x] = (float)npx;
}

int c3_bands(const ConvGeom &g) { return (g.P + TP - 1) / TP; }
int c3_lw(const ConvGeom &g) { return std::max(2 * (g.Q - 1) + 8, g.pw + g.W); }

}  // namespace

bool c3s2_eligible(const ConvGeom &g)
{
    // 14 pixel blocks of 32 must cover TP output rows; the filter row (R taps of 8 x 4)
    // and the staged rows must fit LDS with two workgroups per CU.
    return g.C == 3 && g.K == KOUT && g.sh == 2 && g.sw == 2 && g.R >= 1 && g.R <= 7 && g.S >= 1 && g.S <= 8 &&
           g.W % 8 == 0 && TP * g.Q <= 32 * NBLK && (g.pw % 2) == 1 && c3_lw(g) - g.W <= 16 &&
           c3s2_lds_bytes(g) <= 80 * 1024 &&
           (size_t)g.N * g.P * g.Q * KOUT * 2 < 0x7fffffffu;
}

int c3s2_grid(const ConvGeom &g) { return g.N * c3_bands(g); }

size_t c3s2_lds_bytes(const ConvGeom &g)
{
    const int NR = 2 * (TP - 1) + g.R;
    const size_t stage = (size_t)KOUT * (g.R * 64 + 16) + (size_t)NR * c3_lw(g) * 8;
    const size_t zstage = (size_t)32 * NBLK * KOUT * 2;   // every pixel block of a band
    return std::max({stage, zstage, (size_t)32 * NT * 4});
}

size_t c3s2_wexp_bytes(const ConvGeom &g) { return (size_t)KOUT * g.R * 32 * 2; }

hipError_t launch_conv_c3s2_stats(const ConvGeom &g, const uint16_t *x, const uint16_t *w, uint16_t *wexp,
                                  uint16_t *z, float *partials, hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    hipError_t e = launch(widen_filter_c3_kernel, dim3((KOUT * g.R * 32 + NT - 1) / NT), dim3(NT), 0, st, e0, nullptr,
                          w, g.R, g.S, wexp);
    if (e != hipSuccess) return e;
    C3Params prm;
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
    prm.bands = c3_bands(g);
    prm.LW = c3_lw(g);
    prm.RB = prm.LW * 8;
    prm.WRB = g.R * 64 + 16;
    const size_t lds = c3s2_lds_bytes(g);
    static bool attr_set = false;
    if (!attr_set) {
        e = hipFuncSetAttribute((const void *)conv_c3s2_stats_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                80 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    return launch(conv_c3s2_stats_kernel, dim3(c3s2_grid(g)), dim3(NT), (uint32_t)lds, st, nullptr, e1, prm);
}

}  // namespace cbr
