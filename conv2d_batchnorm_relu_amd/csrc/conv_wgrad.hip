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

struct WgradParams {
    ConvGeom g;
    const uint16_t *dz;
    const uint16_t *x;
    float *out;            // [splits][K][Kg] (or dw itself when splits == 1)
    int rows_per_split;
};

__device__ __forceinline__ int swz(int row, int m)   // element offset of (row, m) in a tile row
{
    return row * LDK + ((((m >> 3) ^ (row >> 3)) & 7) << 3) + (m & 7);
}

template <int BMK, int BNC, bool VEC>
__global__ __launch_bounds__(NT) void conv_wgrad_kernel(WgradParams prm)
{
    constexpr int WM = BMK / 2, WN = BNC / 2;
    constexpr int MI = WM / 16, NJ = WN / 16;
    constexpr int AI = (BKM / 2) * (BMK / 8) / NT;   // (pixel pair, chunk) items per thread
    constexpr int BI = (BKM / 2) * (BNC / 8) / NT;
    constexpr int STAGE = (BMK + BNC) * LDK;
    static_assert(AI >= 1 && BI >= 1, "tile too small for the thread count");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    const ConvGeom &g = prm.g;
    const uint16_t *__restrict__ dz = prm.dz;
    const uint16_t *__restrict__ x = prm.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int k0 = blockIdx.y * BMK, n0 = blockIdx.x * BNC;
    const int mbeg = blockIdx.z * prm.rows_per_split;
    const int mend = min(g.M, mbeg + prm.rows_per_split);
    const int PQ = g.P * g.Q;

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

    u32x4 ra[AI][2], rb[BI][2];
    auto load = [&](int mstep) {
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int it = tid + NT * j;
            const int k = k0 + 8 * item_c(it);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int m = mstep + 2 * item_p(it) + h;
                ra[j][h] = (m < mend && k < g.K) ? *(const u32x4 *)(dz + (size_t)m * g.K + k) : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const int it = tid + NT * j;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int m = mstep + 2 * item_p(it) + h;
                u32x4 v = u32x4{0, 0, 0, 0};
                if (m < mend && b_ok[j]) {
                    const int n = m / PQ, rem = m - n * PQ;
                    const int p = rem / g.Q, q = rem - p * g.Q;
                    const int hb = p * g.sh - g.ph, wb = q * g.sw - g.pw;
                    const uint16_t *xn = x + (size_t)n * g.H * g.W * g.C;
                    if constexpr (VEC) {
                        const int hh = hb + b_r[j], ww = wb + b_s[j];
                        if ((unsigned)hh < (unsigned)g.H && (unsigned)ww < (unsigned)g.W)
                            v = *(const u32x4 *)(xn + (hh * g.W + ww) * g.C + b_c[j]);
                    } else {
                        const int kk0 = n0 + 8 * item_c(it);
                        uint32_t e16[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int kk = kk0 + e;
                            e16[e] = 0u;
                            if (kk < g.Kg) {
                                const int tap = kk / g.C, c = kk - tap * g.C;
                                const int r = tap / g.S, s = tap - r * g.S;
                                const int hh = hb + r, ww = wb + s;
                                if ((unsigned)hh < (unsigned)g.H && (unsigned)ww < (unsigned)g.W)
                                    e16[e] = xn[(hh * g.W + ww) * g.C + c];
                            }
                        }
                        v = u32x4{e16[0] | (e16[1] << 16), e16[2] | (e16[3] << 16), e16[4] | (e16[5] << 16),
                                  e16[6] | (e16[7] << 16)};
                    }
                }
                rb[j][h] = v;
            }
        }
    };
    // Transposed store: channel-chunk element e of pixels (2p, 2p+1) -> row 8*cc + e,
    // columns 2p and 2p+1 (one 32-bit LDS write).
    auto store = [&](int buf) {
        uint16_t *sa = smem + buf * STAGE;
        uint16_t *sb = sa + BMK * LDK;
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int it = tid + NT * j, p = item_p(it), cc = item_c(it);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t lo = (ra[j][0][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                const uint32_t hi = (ra[j][1][e >> 1] >> (16 * (e & 1))) & 0xffffu;
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

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const uint16_t *sa = smem + buf * STAGE;
        const uint16_t *sb = sa + BMK * LDK;
#pragma unroll
        for (int kh = 0; kh < BKM / 32; ++kh) {
            const int mb = kh * 32 + (lane >> 4) * 8;
            bf16x8 a[MI], b[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i) a[i] = *(const bf16x8 *)(sa + swz(wm * WM + 16 * i + (lane & 15), mb));
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[j] = *(const bf16x8 *)(sb + swz(wn * WN + 16 * j + (lane & 15), mb));
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    const int nsteps = (mend - mbeg + BKM - 1) / BKM;
    if (nsteps > 0) {
        load(mbeg);
        store(0);
    }
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int cur = st & 1;
        if (st + 1 < nsteps) load(mbeg + (st + 1) * BKM);
        compute(cur);
        if (st + 1 < nsteps) store(cur ^ 1);
        __syncthreads();
    }

    float *out = prm.out + (size_t)blockIdx.z * g.K * g.Kg;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int k = k0 + wm * WM + 16 * i + 4 * (lane >> 4) + v;
                const int kk = n0 + wn * WN + 16 * j + (lane & 15);
                if (k < g.K && kk < g.Kg) out[(size_t)k * g.Kg + kk] = acc[i][j][v];
            }
}

// dw[i] = sum over splits s (in order) of part[s][i].
__global__ __launch_bounds__(NT) void split_sum_kernel(const float *__restrict__ part, int splits, long n,
                                                       float *__restrict__ dw)
{
    for (long i = (long)blockIdx.x * NT + threadIdx.x; i < n; i += (long)gridDim.x * NT) {
        float s = 0.f;
        for (int t = 0; t < splits; ++t) s += part[(size_t)t * n + i];
        dw[i] = s;
    }
}

// Filter of the data gradient as a forward convolution (stride 1):
// wt[c][r'][s'][k] = w[k][R-1-r'][S-1-s'][c].
__global__ __launch_bounds__(NT) void flip_weights_kernel(const uint16_t *__restrict__ w, int K, int R, int S, int C,
                                                          uint16_t *__restrict__ wt)
{
    const long total = (long)K * R * S * C;
    for (long i = (long)blockIdx.x * NT + threadIdx.x; i < total; i += (long)gridDim.x * NT) {
        long t = i;
        const int k = (int)(t % K); t /= K;
        const int s = (int)(t % S); t /= S;
        const int r = (int)(t % R); t /= R;
        const int c = (int)t;
        wt[i] = w[(((size_t)k * R + (R - 1 - r)) * S + (S - 1 - s)) * C + c];
    }
}

}  // namespace

WgradPlan wgrad_plan(int M, int K, int Kg)
{
    WgradPlan p;
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

hipError_t launch_conv_wgrad(const ConvGeom &g, const uint16_t *dz, const uint16_t *x, float *part, float *dw,
                             hipStream_t st, hipEvent_t e0, hipEvent_t e1)
{
    const WgradPlan p = wgrad_plan(g.M, g.K, g.Kg);
    WgradParams prm{g, dz, x, p.splits == 1 ? dw : part, p.rows_per_split};
    dim3 grid(p.tiles_n, p.tiles_m, p.splits);
    const bool vec = (g.C % 8) == 0;
    const hipEvent_t ek = p.splits == 1 ? e1 : nullptr;   // end event on the last kernel of the stage
    hipError_t e;
    if (p.bm == 128)
        e = vec ? launch(conv_wgrad_kernel<128, 128, true>, grid, dim3(NT), 0, st, e0, ek, prm)
                : launch(conv_wgrad_kernel<128, 128, false>, grid, dim3(NT), 0, st, e0, ek, prm);
    else
        e = vec ? launch(conv_wgrad_kernel<64, 128, true>, grid, dim3(NT), 0, st, e0, ek, prm)
                : launch(conv_wgrad_kernel<64, 128, false>, grid, dim3(NT), 0, st, e0, ek, prm);
    if (e != hipSuccess || p.splits == 1) return e;
    const long n = (long)g.K * g.Kg;
    const int blocks = (int)std::min<long>((n + NT - 1) / NT, 8192);
    return launch(split_sum_kernel, dim3(blocks), dim3(NT), 0, st, nullptr, e1, (const float *)part, p.splits, n, dw);
}

hipError_t launch_flip_weights(int K, int R, int S, int C, const uint16_t *w, uint16_t *wt, hipStream_t st,
                               hipEvent_t e0, hipEvent_t e1)
{
    const long total = (long)K * R * S * C;
    const int blocks = (int)std::min<long>((total + NT - 1) / NT, 4096);
    return launch(flip_weights_kernel, dim3(blocks), dim3(NT), 0, st, e0, e1, w, K, R, S, C, wt);
}

}  // namespace cbr
