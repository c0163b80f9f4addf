// MoE MLP with router replay for the grouped decode step
// (gist.science/es/paper/2608.12385, "Mecanismos Clave": in MoE models the
// aux flow reuses the set of experts the primary router picked, applying
// them with its own mixture weights).
//
// 1. moe_route (one workgroup): the primary ranking per sequence
//    (descending logit, ties to the lower expert id), softmax gates of each
//    flow over its fan-out (k primary ranks; the aux flow may take more or
//    fewer of the primary's ranks: independent fan-outs, "Contribuciones
//    Clave" item 3), then a stable counting sort of the (sequence, rank)
//    pairs by expert: offsets[E+1], perm (sorted slot -> pair), inv.
// 2. moe_expert (up): one workgroup per (expert, 32 rows of the expert FFN);
//    the expert's stacked rows are the primary and aux rows of its pairs, so
//    each touched expert's weights are read once for both flows; untouched
//    experts exit without reading. Epilogue: GELU, then the b coupling on the
//    aux row where the primary also ran that expert.
// 3. moe_expert (down): same grouping over the expert's down projection.
// 4. moe_combine: gate-weighted sum over each flow's ranks in rank order, c
//    coupling on the aux output, residual add, then the next LayerNorm of the
//    updated rows. Integer work (ids, offsets, perm) is exact; no atomics.
#include <algorithm>

#include "df_device.h"
#include "df_internal.h"
#include "mfma_tile.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

using tile::f32x4;
using tile::RT;
using tile::ROWS;

constexpr int kMaxK = 16;

// Routing: the primary ranking (top-kr of the primary router logits by
// descending value, ties to the lower id), gates of each flow over its
// fan-out (primary: the first k ranks, aux: the first ka), then a stable
// counting sort of the (sequence, rank) pairs in use by expert. kk ranks per
// sequence are in use: kr with both flows, k for the primary alone.
// One workgroup of 1024 threads: wave w ranks sequences w, w + 16, ... by kr
// rounds of a wave-wide argmax over the logits held in registers (E <= 1024,
// 16 per lane); then thread e counts expert e's pairs, thread t places pair t.
constexpr int kRouteThreads = 1024;
constexpr int kPerLane = 16;   // E <= 64 * kPerLane

template <int NPL>   // logits per lane: E <= 64 NPL
__global__ __launch_bounds__(kRouteThreads) void moe_route(const float* r, const float* r1_given, int B, int E,
                                                           int k, int ka, int nflows, int32_t* ids, float* gates,
                                                           int32_t* ids_out, int32_t* offsets, int32_t* perm,
                                                           int32_t* inv) {
    __shared__ int32_t s_ids[64 * kMaxK];
    __shared__ int32_t s_cnt[1024];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    constexpr int NWAVE = kRouteThreads / 64, SPW = 64 / NWAVE;   // sequences per wave (B <= 64)
    const int kr = max(k, ka), kk = nflows == 2 ? kr : k;
    // every logit row of the wave's sequences first (both flows): one memory
    // latency for all; the SPW sequences are then ranked side by side, so
    // their shuffle chains overlap
    float v[SPW][NPL], w2[SPW][NPL];
    const int nper = (E + 63) / 64;   // logits per lane in use
    #pragma unroll
    for (int q = 0; q < SPW; ++q) {
        const int b = wv + NWAVE * q;
        const float* r1 = r1_given ? r1_given + (size_t)b * E : r + (size_t)(2 * b) * E;
        const float* r2 = r + (size_t)(2 * b + 1) * E;
        #pragma unroll
        for (int i = 0; i < NPL; ++i) {
            const int e = lane + 64 * i;
            const bool ok = b < B && e < E;
            v[q][i] = ok ? r1[e] : -INFINITY;
            w2[q][i] = (ok && nflows == 2) ? r2[e] : -INFINITY;
        }
    }
    unsigned taken[SPW];
    float my_val[SPW];
    int my_sel[SPW];   // lane j ends with rank j's expert and logit
    #pragma unroll
    for (int q = 0; q < SPW; ++q) { taken[q] = 0; my_val[q] = -INFINITY; my_sel[q] = 0; }
    for (int j = 0; j < kr; ++j) {
        float bv[SPW];
        int bi[SPW];
        #pragma unroll
        for (int q = 0; q < SPW; ++q) {   // lane-local best (largest value, then lowest id)
            bv[q] = -INFINITY;
            bi[q] = 0x7fffffff;
            #pragma unroll
            for (int i = 0; i < NPL; ++i) {
                const int e = lane + 64 * i;
                if (i < nper && e < E && !((taken[q] >> i) & 1u) && (v[q][i] > bv[q] || bi[q] == 0x7fffffff)) {
                    bv[q] = v[q][i];
                    bi[q] = e;
                }
            }
        }
        for (int o = 32; o > 0; o >>= 1) {   // the wave's best, SPW chains side by side
            #pragma unroll
            for (int q = 0; q < SPW; ++q) {
                const float ov = __shfl_xor(bv[q], o, 64);
                const int oi = __shfl_xor(bi[q], o, 64);
                if (ov > bv[q] || (ov == bv[q] && oi < bi[q])) { bv[q] = ov; bi[q] = oi; }
            }
        }
        #pragma unroll
        for (int q = 0; q < SPW; ++q) {
            if (lane == j) { my_val[q] = bv[q]; my_sel[q] = bi[q]; }
            if ((bi[q] & 63) == lane) taken[q] |= 1u << (bi[q] >> 6);
        }
    }
    // gates: softmax over each flow's ranks (lanes = ranks), zero beyond its fan-out
    #pragma unroll
    for (int q = 0; q < SPW; ++q) {
        const int b = wv + NWAVE * q;
        if (b >= B) break;
        const float top = __shfl(my_val[q], 0, 64);   // rank 0 holds the largest logit
        const float e1 = lane < k ? expf(my_val[q] - top) : 0.f;
        const float s1 = df::wave_sum(e1);
        if (lane < kr) {
            gates[((size_t)b * 2) * kr + lane] = lane < k ? e1 / s1 : 0.f;
            ids[(size_t)b * kr + lane] = my_sel[q];
            if (ids_out) ids_out[(size_t)b * kr + lane] = my_sel[q];
        }
        if (lane < kk) s_ids[b * kk + lane] = my_sel[q];
        if (nflows == 2) {
            // the aux logit of rank `lane`'s expert, from the lane holding it
            float l2 = -INFINITY;
            #pragma unroll
            for (int i = 0; i < NPL; ++i) {
                if (i >= nper) break;
                const float t = __shfl(w2[q][i], my_sel[q] & 63, 64);
                if ((my_sel[q] >> 6) == i) l2 = t;
            }
            l2 = lane < ka ? l2 : -INFINITY;
            const float m2 = df::wave_max(l2);
            const float e2 = lane < ka ? expf(l2 - m2) : 0.f;
            const float s2 = df::wave_sum(e2);
            if (lane < kr) gates[((size_t)b * 2 + 1) * kr + lane] = lane < ka ? e2 / s2 : 0.f;
        }
    }
    __syncthreads();
    // stable counting sort of the P pairs by expert
    const int P = B * kk;
    for (int e = tid; e < E; e += blockDim.x) {
        int c = 0;
        #pragma unroll 8
        for (int t = 0; t < P; ++t) c += (s_ids[t] == e);
        s_cnt[e] = c;
    }
    __syncthreads();
    if (wv == 0) {   // exclusive prefix over the experts: 16 per lane, then across lanes
        int loc[kPerLane], run = 0;
        #pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int e = lane * kPerLane + i;
            loc[i] = run;
            run += e < E ? s_cnt[e] : 0;
        }
        int incl = run;
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, 64);
            if (lane >= o) incl += t;
        }
        const int base = incl - run;
        #pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int e = lane * kPerLane + i;
            if (e < E) { offsets[e] = base + loc[i]; s_cnt[e] = base + loc[i]; }
        }
        if (lane == 63) offsets[E] = incl;
    }
    __syncthreads();
    for (int t = tid; t < P; t += blockDim.x) {
        const int e = s_ids[t];
        int rank = 0;
        #pragma unroll 8
        for (int u = 0; u < t; ++u) rank += (s_ids[u] == e);
        const int slot = s_cnt[e] + rank;
        perm[slot] = t;
        inv[t] = slot;
    }
}

struct ExpParams {
    const float* x;        // up: [2B][d] rows; down: g_rows [P][2][Fe] (fp32)
    const bf16_t* w;       // [E][N][K], each expert matrix in the fragment layout
    int N, K, kk, kp, nflows, kw;   // kk: ranks in use per sequence; kp: primary fan-out
    const int32_t* offsets;
    const int32_t* perm;
    const float* cpl_b;
    float* g_out;          // up: [P][2][Fe]
    float* y_out;          // down: [P][2][d]
    bool up;
};

// Stacked row m of an expert: slot s = off + m / nflows, flow f = m % nflows.
template <int MT, int KU>
__global__ __launch_bounds__(1024) void moe_expert(ExpParams p) {
    extern __shared__ float red[];
    const int e = blockIdx.y;
    const int off = p.offsets[e], cnt = p.offsets[e + 1] - off;
    if (cnt == 0) return;   // untouched expert: its weights are never read
    const int M = cnt * p.nflows;
    const int mtiles = min((M + 15) / 16, MT);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, NW = blockDim.x >> 6;
    const int n0 = blockIdx.x * ROWS;
    const int li = lane & 15, lg = lane >> 4;
    const bf16_t* W = p.w + (size_t)e * p.N * p.K;
    const bf16_t* wrow[RT];
    #pragma unroll
    for (int rt = 0; rt < RT; ++rt) wrow[rt] = tile::frag_tile(W, min(n0 / 16 + rt, p.N / 16 - 1), p.K, lane);
    // Several passes when one expert holds more than MT*16 stacked rows.
    for (int mbase = 0; mbase < M; mbase += MT * 16) {
        const int mt_here = min((M - mbase + 15) / 16, mtiles);
        const float* xrow[MT];
        #pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = min(mbase + mt * 16 + li, M - 1);
            const int s = off + m / p.nflows, f = m - (m / p.nflows) * p.nflows;
            size_t row;
            if (p.up) row = (size_t)(2 * (p.perm[s] / p.kk) + f);   // sequence b = pair / kk
            else row = (size_t)s * 2 + f;                         // g_rows[slot][flow]
            xrow[mt] = p.x + row * p.K + lg * 8;
        }
        f32x4 acc[RT][MT];
        tile::zero<MT>(acc);
        tile::stream_k<MT, KU>(wrow, xrow, mt_here, wv * p.kw, (wv + 1) * p.kw, acc);
        __syncthreads();
        tile::to_lds<MT>(red, wv, lane, acc);
        __syncthreads();
        const int npairs = min(cnt - mbase / p.nflows, MT * 16 / p.nflows);
        for (int t = threadIdx.x; t < ROWS * npairs; t += blockDim.x) {
            const int nl = t % ROWS, q = t / ROWS;
            const int n = n0 + nl;
            if (n >= p.N) continue;
            const int ml = q * p.nflows;   // local stacked row of the primary
            const float y1 = tile::lds_sum<MT>(red, NW, nl, ml);
            const float y2 = p.nflows == 2 ? tile::lds_sum<MT>(red, NW, nl, ml + 1) : 0.f;
            const int s = off + mbase / p.nflows + q;
            if (p.up) {
                const float g1 = 0.5f * y1 * (1.0f + erff(y1 * 0.70710678118654752f));
                p.g_out[((size_t)s * 2) * p.N + n] = g1;
                if (p.nflows == 2) {
                    float g2 = 0.5f * y2 * (1.0f + erff(y2 * 0.70710678118654752f));
                    // intermediate coupling b_l, per expert the primary also ran (rank < kp)
                    if (p.cpl_b && p.perm[s] % p.kk < p.kp) g2 = fmaf(p.cpl_b[n], g1, g2);
                    p.g_out[((size_t)s * 2 + 1) * p.N + n] = g2;
                }
            } else {
                p.y_out[((size_t)s * 2) * p.N + n] = y1;
                if (p.nflows == 2) p.y_out[((size_t)s * 2 + 1) * p.N + n] = y2;
            }
        }
    }
}

// y_1[b] = sum_{j < k} gate_1[b][j] * y(slot of (b, j))_1, y_2 likewise over
// j < ka; y2 += c * y1; h += y.
// One workgroup per sequence: both flows' gate-weighted sums over their
// ranks (rank order), the c coupling, the residual add; then, with g_next,
// the LayerNorm of the updated rows into x_next (the next projection's
// input), the rows being at hand.
constexpr int kCombThreads = 1024;
constexpr int kCombCols = 4;   // d <= kCombThreads * kCombCols
__global__ __launch_bounds__(kCombThreads) void moe_combine(const float* y_rows, const float* gates, const int32_t* inv,
                                                            const float* cpl_c, int d, int k, int ka, int kr, int kk,
                                                            int nflows, float* h, const float* g_next, float eps,
                                                            float* x_next) {
    __shared__ int s_slot[kMaxK];
    __shared__ float s_g[2][kMaxK];
    __shared__ float red[16];
    const int b = blockIdx.x, tid = threadIdx.x;
    const bool dual = nflows == 2;
    if (tid < kk) s_slot[tid] = inv[(size_t)b * kk + tid];
    if (tid < kr) {
        s_g[0][tid] = gates[((size_t)b * 2) * kr + tid];
        s_g[1][tid] = dual ? gates[((size_t)b * 2 + 1) * kr + tid] : 0.f;
    }
    __syncthreads();
    float v1[kCombCols], v2[kCombCols];
    float s1 = 0.f, s2 = 0.f;
    #pragma unroll
    for (int c = 0; c < kCombCols; ++c) {
        const int n = tid + kCombThreads * c;
        v1[c] = v2[c] = 0.f;
        if (n >= d) continue;
        float y1 = 0.f, y2 = 0.f;
        for (int j = 0; j < k; ++j) y1 = fmaf(s_g[0][j], y_rows[((size_t)s_slot[j] * 2) * d + n], y1);
        if (dual)
            for (int j = 0; j < ka; ++j) y2 = fmaf(s_g[1][j], y_rows[((size_t)s_slot[j] * 2 + 1) * d + n], y2);
        float* h1 = h + (size_t)(2 * b) * d + n;
        v1[c] = *h1 + y1;
        *h1 = v1[c];
        s1 += v1[c];
        if (dual) {
            if (cpl_c) y2 = fmaf(cpl_c[n], y1, y2);   // output coupling c_l
            float* h2 = h1 + d;
            v2[c] = *h2 + y2;
            *h2 = v2[c];
            s2 += v2[c];
        }
    }
    if (!x_next) return;
    const float mean1 = df::block_sum(s1, red) / (float)d;
    const float mean2 = dual ? df::block_sum(s2, red) / (float)d : 0.f;
    float q1 = 0.f, q2 = 0.f;
    #pragma unroll
    for (int c = 0; c < kCombCols; ++c) {
        if (tid + kCombThreads * c >= d) continue;
        q1 = fmaf(v1[c] - mean1, v1[c] - mean1, q1);
        q2 = fmaf(v2[c] - mean2, v2[c] - mean2, q2);
    }
    const float rstd1 = 1.0f / sqrtf(df::block_sum(q1, red) / (float)d + eps);
    const float rstd2 = dual ? 1.0f / sqrtf(df::block_sum(q2, red) / (float)d + eps) : 0.f;
    #pragma unroll
    for (int c = 0; c < kCombCols; ++c) {
        const int n = tid + kCombThreads * c;
        if (n >= d) continue;
        x_next[(size_t)(2 * b) * d + n] = (v1[c] - mean1) * rstd1 * g_next[n];
        if (dual) x_next[(size_t)(2 * b + 1) * d + n] = (v2[c] - mean2) * rstd2 * g_next[n];
    }
}

template <int MT>
hipError_t launch_expert(ExpParams& p, int E, hipStream_t s) {
    constexpr int KU = 2;
    const int nwg = (p.N + ROWS - 1) / ROWS;
    const int nw = tile::pick_waves(nwg * E, p.K, MT, KU, 8192);
    p.kw = p.K / nw;
    const size_t lds = (size_t)nw * RT * MT * 256 * sizeof(float);
    hipError_t e = tile::allow_lds(reinterpret_cast<const void*>(&moe_expert<MT, KU>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((moe_expert<MT, KU>), dim3(nwg, E), dim3(64 * nw), lds, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t moe(const MoeArgs& a, hipStream_t s) {
    const int ka = a.ka > 0 ? a.ka : a.k;
    const int kr = std::max(a.k, ka), kk = a.nflows == 2 ? kr : a.k;
    if (kr > kMaxK || a.B > 64 || a.E > 64 * kPerLane || a.dtype != DF_BF16) return hipErrorInvalidValue;
    (void)hipGetLastError();
    const auto route = a.E <= 64 ? moe_route<1> : a.E <= 256 ? moe_route<4> : moe_route<kPerLane>;
    hipLaunchKernelGGL(route, dim3(1), dim3(kRouteThreads), 0, s, a.r, a.r1_given, a.B, a.E, a.k, ka, a.nflows,
                       a.ids, a.gates, a.ids_out, a.offsets, a.perm, a.inv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ExpParams up;
    up.x = a.x;
    up.w = reinterpret_cast<const bf16_t*>(a.w_up);
    up.N = a.Fe; up.K = a.d; up.kk = kk; up.kp = a.k; up.nflows = a.nflows; up.offsets = a.offsets; up.perm = a.perm;
    up.cpl_b = a.cpl_b; up.g_out = a.g_rows; up.y_out = nullptr; up.up = true;
    e = launch_expert<2>(up, a.E, s);
    if (e != hipSuccess) return e;
    ExpParams dn = up;
    dn.x = a.g_rows;
    dn.w = reinterpret_cast<const bf16_t*>(a.w_down);
    dn.N = a.d; dn.K = a.Fe; dn.g_out = nullptr; dn.y_out = a.y_rows; dn.up = false;
    e = launch_expert<2>(dn, a.E, s);
    if (e != hipSuccess) return e;
    if (a.d > kCombThreads * kCombCols) return hipErrorInvalidValue;
    hipLaunchKernelGGL(moe_combine, dim3(a.B), dim3(kCombThreads), 0, s, a.y_rows, a.gates, a.inv, a.cpl_c, a.d, a.k,
                       ka, kr, kk, a.nflows, a.h, a.g_next, a.eps, a.x_next);
    return hipGetLastError();
}

}  // namespace dfk
