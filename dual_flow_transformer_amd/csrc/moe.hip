// MoE MLP with router replay for the grouped decode step
// (gist.science/es/paper/2608.12385, "Mecanismos Clave": in MoE models the
// aux flow reuses the set of experts the primary router picked, applying
// them with its own mixture weights).
//
// 1. moe_gate (one workgroup per sequence): LayerNorm of the sequence's
//    stacked rows, the router logits of each row, the primary ranking
//    (descending logit, ties to the lower expert id) and the softmax gates
//    of each flow over its fan-out (k primary ranks; the aux flow may take
//    more or fewer of the primary's ranks: independent fan-outs,
//    "Contribuciones Clave" item 3).
// 2. moe_expert (up): one workgroup per (expert, 32 rows of the expert FFN);
//    it finds the (sequence, rank) pairs that chose its expert, in pair
//    order, and stacks their primary and aux rows, so each touched expert's
//    weights are read once for both flows; untouched experts exit without
//    reading. Epilogue: GELU, then the b coupling on the aux row where the
//    primary also ran that expert. Outputs are indexed by pair.
// 3. moe_expert (down): same grouping over the expert's down projection.
// 4. moe_combine: gate-weighted sum over each flow's ranks in rank order, c
//    coupling on the aux output, residual add, then the next LayerNorm of the
//    updated rows. Integer work (ids, pair lists) is exact; no atomics.
#include <algorithm>

#include "df_device.h"
#include "df_internal.h"
#include "mfma_tile.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

using tile::f32x4;
using tile::u32x4;
using tile::RT;
using tile::ROWS;

constexpr int kMaxK = 16;
constexpr int kPerLane = 16;   // E <= 64 * kPerLane

// Router of one sequence per workgroup: LayerNorm of its stacked rows from
// their per-segment statistics (to x, the experts' input, and to LDS), the
// router logits of each row, then on wave 0 the primary ranking (kr rounds
// of a wave-wide argmax over the logits held in registers, NPL per lane)
// and the gates of both flows. Logits: item (16-expert group g, k-split q)
// goes to one wave, whose lane l reads 16 B of each 1 KiB weight fragment
// of the item (expert 16 g + l % 16, k = 32 kb + 8 (l / 16) + i); all of a
// wave's weight loads are issued before the LayerNorm, so the two overlap.
// The four lanes of an expert, then its k-splits in order, are added.
struct GateParams {
    const float* h;          // [2B][d] residual rows
    const float* stats;      // their per-segment statistics
    const float* g;          // LN gain [d]
    float eps;
    int d, E, k, ka, kr, nflows;
    int ns;                  // k-splits per 16-expert group
    const bf16_t* wr;        // router [E][d], fragment layout
    const float* r1_given;   // [B][E] primary logits supplied, or nullptr
    float* x;                // [2B][d] LN(h) rows
    int32_t* ids;            // [B][kr]
    float* gates;            // [B][2][kr], zero beyond a flow's fan-out
    int32_t* ids_out;        // [B][kr] or nullptr
};
constexpr int kGateThreads = 1024;
constexpr int kGateWaves = kGateThreads / 64;
constexpr int kGateFrags = 16;   // weight fragments per lane in flight

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}

// (v, i) := the better of (v, i) and (ov, oi): larger value, then lower index.
__device__ __forceinline__ void take_best(float& v, int& i, float ov, int oi) {
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

// Wave-wide best (largest value, then lowest index); every lane ends with
// it. A total order, so the reduction tree does not change the result:
// quad, half-row and row exchanges by DPP, then two cross-row shuffles.
__device__ __forceinline__ void wave_best(float& v, int& i) {
    take_best(v, i, df::dpp<df::kQuadSwap1>(v), dpp_i<df::kQuadSwap1>(i));
    take_best(v, i, df::dpp<df::kQuadSwap2>(v), dpp_i<df::kQuadSwap2>(i));
    take_best(v, i, df::dpp<df::kRowHalfMirror>(v), dpp_i<df::kRowHalfMirror>(i));
    take_best(v, i, df::dpp<df::kRowMirror>(v), dpp_i<df::kRowMirror>(i));
    take_best(v, i, __shfl_xor(v, 16, 64), __shfl_xor(i, 16, 64));
    take_best(v, i, __shfl_xor(v, 32, 64), __shfl_xor(i, 32, 64));
}

template <int NPL>   // logits per lane: E <= 64 NPL
__global__ __launch_bounds__(kGateThreads) void moe_gate(GateParams p) {
    extern __shared__ float s_x[];   // [2][d] normalised rows, then [2][E / 16][ns][16] logit parts
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int d = p.d, E = p.E, nseg = stat_segs(d), KB = d / 32, ns = p.ns, kbs = KB / ns;
    const int items = (E / 16) * ns;
    float* s_part = s_x + 2 * d;
    const bool dual = p.nflows == 2;
    // first chunk of the wave's first item: loads in flight during the norm
    int it = wv;
    u32x4 w[kGateFrags];
    auto load = [&](int item, int kb0) {
        const int grp = min(item, items - 1) / ns;
        const int q = min(item, items - 1) - grp * ns;
        const bf16_t* wp = p.wr + ((size_t)(grp * KB + q * kbs) * 64 + lane) * 8;
        #pragma unroll
        for (int u = 0; u < kGateFrags; ++u)
            w[u] = *reinterpret_cast<const u32x4*>(wp + (size_t)min(kb0 + u, kbs - 1) * 512);
    };
    load(it, 0);
    {
        // residual values of both rows (one float4 per thread and row:
        // d <= 4 * kGateThreads) and the gains, in flight while wave 0 forms
        // the row norms: lane 16 f + i loads segment i of row f, and each
        // 16-lane group combines its segments' (mean, M2) (Chan), as the
        // projections' on-the-fly LayerNorm does
        __shared__ float2 s_mr[2];
        const int k = min(tid * 4, d - 4);
        float4 hv[2];
        #pragma unroll
        for (int f = 0; f < 2; ++f)
            hv[f] = *reinterpret_cast<const float4*>(p.h + (size_t)(2 * b + (dual ? f : 0)) * d + k);
        const float4 gv = *reinterpret_cast<const float4*>(p.g + k);
        if (wv == 0) {
            const int f = (lane >> 4) & 1, i = lane & 15;
            const float2 sv = reinterpret_cast<const float2*>(p.stats)[(size_t)(2 * b + (dual ? f : 0)) * nseg +
                                                                        min(i, nseg - 1)];
            const bool valid = i < nseg;
            const float cnt = valid ? (float)min(kStatSeg, d - i * kStatSeg) : 0.f;
            const float mean = df::group_sum<16>(cnt * sv.x) / (float)d;
            const float dm = sv.x - mean;
            const float m2 = df::group_sum<16>(valid ? fmaf(cnt * dm, dm, sv.y) : 0.f);
            if (lane < 32 && i == 0) s_mr[f] = make_float2(mean, 1.0f / sqrtf(m2 / (float)d + p.eps));
        }
        __syncthreads();
        #pragma unroll
        for (int f = 0; f < 2; ++f) {
            if (f >= p.nflows || tid * 4 >= d) break;
            const float2 mr = s_mr[f];
            const float4 h4 = hv[f];
            const float4 v = make_float4((h4.x - mr.x) * mr.y * gv.x, (h4.y - mr.x) * mr.y * gv.y,
                                         (h4.z - mr.x) * mr.y * gv.z, (h4.w - mr.x) * mr.y * gv.w);
            *reinterpret_cast<float4*>(p.x + (size_t)(2 * b + f) * d + k) = v;
            *reinterpret_cast<float4*>(s_x + f * d + k) = v;
        }
    }
    __syncthreads();
    for (; it < items; it += kGateWaves) {
        const int grp = it / ns, q = it - (it / ns) * ns;
        const float* x1 = s_x + 32 * q * kbs + 8 * (lane >> 4);
        const float* x2 = x1 + d;
        float a1 = 0.f, a2 = 0.f;
        for (int kb0 = 0; kb0 < kbs; kb0 += kGateFrags) {
            if (kb0 > 0) load(it, kb0);
            #pragma unroll
            for (int u = 0; u < kGateFrags; ++u) {
                if (kb0 + u >= kbs) break;
                const int kb = kb0 + u;
                const float wf[8] = {df::bf16_lo(w[u][0]), df::bf16_hi(w[u][0]), df::bf16_lo(w[u][1]),
                                     df::bf16_hi(w[u][1]), df::bf16_lo(w[u][2]), df::bf16_hi(w[u][2]),
                                     df::bf16_lo(w[u][3]), df::bf16_hi(w[u][3])};
                #pragma unroll
                for (int i = 0; i < 8; ++i) a1 = fmaf(wf[i], x1[32 * kb + i], a1);
                if (dual) {
                    #pragma unroll
                    for (int i = 0; i < 8; ++i) a2 = fmaf(wf[i], x2[32 * kb + i], a2);
                }
            }
        }
        a1 += __shfl_xor(a1, 16, 64);
        a1 += __shfl_xor(a1, 32, 64);
        a2 += __shfl_xor(a2, 16, 64);
        a2 += __shfl_xor(a2, 32, 64);
        if (lane < 16) {
            s_part[(grp * ns + q) * 16 + lane] = a1;
            s_part[(items + grp * ns + q) * 16 + lane] = a2;
        }
        if (it + kGateWaves < items) load(it + kGateWaves, 0);
    }
    __syncthreads();
    // logits of both rows (k-splits in order) into the first 2 E floats of
    // LDS, once every part has been read (E <= kGateThreads)
    float l1 = 0.f, l2 = 0.f;
    const int e = tid;
    if (e < E) {
        const int grp = e / 16, j = e - (e / 16) * 16;
        for (int q = 0; q < ns; ++q) {
            l1 += s_part[(grp * ns + q) * 16 + j];
            l2 += s_part[(items + grp * ns + q) * 16 + j];
        }
    }
    __syncthreads();
    float* s_r = s_x;
    if (e < E) { s_r[e] = l1; s_r[E + e] = l2; }
    __syncthreads();
    if (wv != 0) return;
    const float* r1 = p.r1_given ? p.r1_given + (size_t)b * E : s_r;
    float v[NPL];
    #pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? r1[e] : -INFINITY;
    }
    unsigned taken = 0;
    float my_val = -INFINITY;
    int my_sel = 0;   // lane j ends with rank j's expert and logit
    for (int j = 0; j < p.kr; ++j) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        #pragma unroll
        for (int i = 0; i < NPL; ++i) {   // lane-local best (largest value, then lowest id)
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && (v[i] > bv || bi == 0x7fffffff)) {
                bv = v[i];
                bi = e;
            }
        }
        wave_best(bv, bi);
        if (lane == j) { my_val = bv; my_sel = bi; }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
    // gates: softmax over each flow's ranks (lanes = ranks), zero beyond its fan-out
    const float top = __shfl(my_val, 0, 64);   // rank 0 holds the largest logit
    const float e1 = lane < p.k ? expf(my_val - top) : 0.f;
    const float s1 = df::wave_sum(e1);
    if (lane < p.kr) {
        p.gates[((size_t)b * 2) * p.kr + lane] = lane < p.k ? e1 / s1 : 0.f;
        p.ids[(size_t)b * p.kr + lane] = my_sel;
        if (p.ids_out) p.ids_out[(size_t)b * p.kr + lane] = my_sel;
    }
    if (dual) {
        // the aux router's logit of rank `lane`'s expert
        const float l2 = lane < p.ka ? s_r[E + my_sel] : -INFINITY;
        const float m2 = df::wave_max(l2);
        const float e2 = lane < p.ka ? expf(l2 - m2) : 0.f;
        const float s2 = df::wave_sum(e2);
        if (lane < p.kr) p.gates[((size_t)b * 2 + 1) * p.kr + lane] = lane < p.ka ? e2 / s2 : 0.f;
    }
}

// The pairs t = b kk + j (rank j < kk of sequence b) whose expert is e, in
// increasing t, into s_pairs (at most one per sequence: a sequence's ranks
// are distinct experts); returns their count. Ballots per wave, then the
// counts of the lower waves.
constexpr int kMaxPairs = 64;   // sequences per step at most
__device__ int expert_pairs(const int32_t* ids, int kr, int kk, int P, int e, int* s_pairs, int* s_wc) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int base = 0;
    for (int t0 = 0; t0 < P; t0 += blockDim.x) {
        const int t = t0 + threadIdx.x;
        const bool hit = t < P && ids[(size_t)(t / kk) * kr + t % kk] == e;
        const unsigned long long m = __ballot(hit);
        if (lane == 0) s_wc[wv] = __popcll(m);
        __syncthreads();
        int before = base, total = base;
        for (int w = 0; w < nw; ++w) {
            before += w < wv ? s_wc[w] : 0;
            total += s_wc[w];
        }
        const int pos = before + __popcll(m & ((1ull << lane) - 1ull));
        if (hit && pos < kMaxPairs) s_pairs[pos] = t;
        __syncthreads();   // s_wc is rewritten by the next chunk
        base = total;
    }
    return min(base, kMaxPairs);
}

struct ExpParams {
    const float* x;        // up: [2B][d] rows; down: g rows [P][2][Fe] (fp32)
    const bf16_t* w;       // [E][N][K], each expert matrix in the fragment layout
    int N, K, kk, kp, nflows, kw;   // kk: ranks in use per sequence; kp: primary fan-out
    const int32_t* ids;    // [B][kr] expert of each rank
    int kr, P;             // ids row length; pairs in use (B kk)
    const float* cpl_b;
    float* g_out;          // up: [P][2][Fe], row 2 t + f
    float* y_out;          // down: [P][2][d], row 2 t + f
    bool up;
};

// Stacked row m of an expert: pair t = s_pairs[m / nflows], flow f = m % nflows.
template <int MT, int KU>
__global__ __launch_bounds__(1024) void moe_expert(ExpParams p) {
    extern __shared__ float red[];
    __shared__ int s_pairs[kMaxPairs];
    __shared__ int s_wc[16];
    const int e = blockIdx.y;
    const int cnt = expert_pairs(p.ids, p.kr, p.kk, p.P, e, s_pairs, s_wc);
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
            const int t = s_pairs[m / p.nflows], f = m - (m / p.nflows) * p.nflows;
            size_t row;
            if (p.up) row = (size_t)(2 * (t / p.kk) + f);   // sequence b = pair / kk
            else row = (size_t)t * 2 + f;                  // g rows [pair][flow]
            xrow[mt] = p.x + row * p.K + lg * 8;
        }
        f32x4 acc[RT][MT];
        tile::zero<MT>(acc);
        tile::stream_k<MT, KU>(wrow, xrow, mt_here, wv * p.kw, (wv + 1) * p.kw, acc);
        __syncthreads();
        tile::to_lds<MT>(red, wv, lane, acc);
        __syncthreads();
        const int npairs = min(cnt - mbase / p.nflows, MT * 16 / p.nflows);
        for (int i = threadIdx.x; i < ROWS * npairs; i += blockDim.x) {
            const int nl = i % ROWS, q = i / ROWS;
            const int n = n0 + nl;
            if (n >= p.N) continue;
            const int ml = q * p.nflows;   // local stacked row of the primary
            const float y1 = tile::lds_sum<MT>(red, NW, nl, ml);
            const float y2 = p.nflows == 2 ? tile::lds_sum<MT>(red, NW, nl, ml + 1) : 0.f;
            const int t = s_pairs[mbase / p.nflows + q];
            if (p.up) {
                const bool cpl = p.cpl_b && p.nflows == 2 && t % p.kk < p.kp;
                const float cb = cpl ? p.cpl_b[n] : 0.f;   // loaded before the first store
                const float g1 = 0.5f * y1 * (1.0f + erff(y1 * 0.70710678118654752f));
                p.g_out[((size_t)t * 2) * p.N + n] = g1;
                if (p.nflows == 2) {
                    float g2 = 0.5f * y2 * (1.0f + erff(y2 * 0.70710678118654752f));
                    // intermediate coupling b_l, per expert the primary also ran (rank < kp)
                    if (cpl) g2 = fmaf(cb, g1, g2);
                    p.g_out[((size_t)t * 2 + 1) * p.N + n] = g2;
                }
            } else {
                p.y_out[((size_t)t * 2) * p.N + n] = y1;
                if (p.nflows == 2) p.y_out[((size_t)t * 2 + 1) * p.N + n] = y2;
            }
        }
    }
}

// y_1[b] = sum_{j < k} gate_1[b][j] * y(pair (b, j))_1, y_2 likewise over
// j < ka; y2 += c * y1; h += y.
// One workgroup per sequence: both flows' gate-weighted sums over their
// ranks (rank order), the c coupling, the residual add; then, with g_next,
// the LayerNorm of the updated rows into x_next (the next projection's
// input), the rows being at hand. Every global load of a thread (the gates
// in lanes 0..kr-1 of each wave, the expert outputs of four ranks, the
// residual rows, coupling and gains) is issued before the first use, so the
// kernel waits on one memory round trip, not a chain of them.
constexpr int kCombMaxThreads = 1024;
constexpr int kCombCols = 4;   // d <= kCombMaxThreads * kCombCols

// Threads of the combine for width d: kCombCols columns each, whole waves.
inline int comb_threads(int d) {
    const int t = (d + kCombCols - 1) / kCombCols;
    return std::min(kCombMaxThreads, std::max(64, (t + 63) / 64 * 64));
}

// Block-wide sums of two values with one pair of barriers (each as
// df::block_sum adds it: the wave's lanes, then the waves in order).
__device__ __forceinline__ float2 block_sum2(float a, float c, float2* red /* >= 16 */) {
    a = df::wave_sum(a);
    c = df::wave_sum(c);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = make_float2(a, c);
    __syncthreads();
    float2 t = make_float2(0.f, 0.f);
    for (int i = 0; i < nw; ++i) {
        t.x += red[i].x;
        t.y += red[i].y;
    }
    return t;
}

__device__ __forceinline__ float lane_value(float v, int j) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

__global__ __launch_bounds__(kCombMaxThreads) void moe_combine(const float* y_rows, const float* gates, const float* cpl_c, int d, int k, int ka, int kr, int kk,
                                                               int nflows, float* h, const float* g_next, float eps,
                                                               float* x_next) {
    __shared__ float2 red[16];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, nt = blockDim.x;
    const bool dual = nflows == 2;
    const int nj = dual ? max(k, ka) : k;
    // gates of rank `lane` of both flows
    const float gl1 = lane < kr ? gates[((size_t)b * 2) * kr + lane] : 0.f;
    const float gl2 = (dual && lane < kr) ? gates[((size_t)b * 2 + 1) * kr + lane] : 0.f;
    // residual rows, coupling and gains of every column
    float h1v[kCombCols], h2v[kCombCols], cv[kCombCols], gv[kCombCols];
    #pragma unroll
    for (int c = 0; c < kCombCols; ++c) {
        const int n = min(tid + nt * c, d - 1);
        h1v[c] = h[(size_t)(2 * b) * d + n];
        h2v[c] = dual ? h[(size_t)(2 * b + 1) * d + n] : 0.f;
        cv[c] = (dual && cpl_c) ? cpl_c[n] : 0.f;
        gv[c] = x_next ? g_next[n] : 0.f;
    }
    // gate-weighted sums, the expert outputs of four ranks at a time (every
    // column of the thread, both flows; pair t = b kk + j holds rows 2 t + f);
    // each sum adds its ranks in rank order
    float y1[kCombCols], y2[kCombCols];
    #pragma unroll
    for (int c = 0; c < kCombCols; ++c) y1[c] = y2[c] = 0.f;
    for (int j0 = 0; j0 < nj; j0 += 4) {
        float t1[4][kCombCols], t2[4][kCombCols];
        #pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t r = ((size_t)b * kk + min(j0 + u, nj - 1)) * 2 * d;
            #pragma unroll
            for (int c = 0; c < kCombCols; ++c) {
                const int n = min(tid + nt * c, d - 1);
                t1[u][c] = y_rows[r + n];
                t2[u][c] = dual ? y_rows[r + d + n] : 0.f;
            }
        }
        #pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + u;
            const float g1 = lane_value(gl1, min(j, 63)), g2 = lane_value(gl2, min(j, 63));
            #pragma unroll
            for (int c = 0; c < kCombCols; ++c) {
                if (j < k) y1[c] = fmaf(g1, t1[u][c], y1[c]);
                if (dual && j < ka) y2[c] = fmaf(g2, t2[u][c], y2[c]);
            }
        }
    }
    float v1[kCombCols], v2[kCombCols];
    float s1 = 0.f, s2 = 0.f;
    #pragma unroll
    for (int c = 0; c < kCombCols; ++c) {
        const int n = tid + nt * c;
        v1[c] = v2[c] = 0.f;
        if (n >= d) continue;
        float* h1 = h + (size_t)(2 * b) * d + n;
        v1[c] = h1v[c] + y1[c];
        *h1 = v1[c];
        s1 += v1[c];
        if (dual) {
            float yy2 = y2[c];
            if (cpl_c) yy2 = fmaf(cv[c], y1[c], yy2);   // output coupling c_l
            v2[c] = h2v[c] + yy2;
            h1[d] = v2[c];
            s2 += v2[c];
        }
    }
    if (!x_next) return;
    const float2 sm = block_sum2(s1, s2, red);
    const float mean1 = sm.x / (float)d;
    const float mean2 = dual ? sm.y / (float)d : 0.f;
    float q1 = 0.f, q2 = 0.f;
    #pragma unroll
    for (int c = 0; c < kCombCols; ++c) {
        if (tid + nt * c >= d) continue;
        q1 = fmaf(v1[c] - mean1, v1[c] - mean1, q1);
        q2 = fmaf(v2[c] - mean2, v2[c] - mean2, q2);
    }
    const float2 sq = block_sum2(q1, q2, red);
    const float rstd1 = 1.0f / sqrtf(sq.x / (float)d + eps);
    const float rstd2 = dual ? 1.0f / sqrtf(sq.y / (float)d + eps) : 0.f;
    #pragma unroll
    for (int c = 0; c < kCombCols; ++c) {
        const int n = tid + nt * c;
        if (n >= d) continue;
        x_next[(size_t)(2 * b) * d + n] = (v1[c] - mean1) * rstd1 * gv[c];
        if (dual) x_next[(size_t)(2 * b + 1) * d + n] = (v2[c] - mean2) * rstd2 * gv[c];
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
    if (kr > kMaxK || a.k < 1 || a.B < 1 || a.B > kMaxPairs || a.E < 16 || a.E % 16 || a.E > 64 * kPerLane ||
        a.d < 32 || a.d % 32 || a.d > kMaxSeg * kStatSeg || a.d > kCombMaxThreads * kCombCols || a.dtype != DF_BF16 ||
        (a.nflows != 1 && a.nflows != 2))
        return hipErrorInvalidValue;
    GateParams gp;
    gp.h = a.h; gp.stats = a.stats; gp.g = a.g_ln; gp.eps = a.eps; gp.d = a.d; gp.E = a.E; gp.k = a.k; gp.ka = ka;
    gp.kr = kr; gp.nflows = a.nflows; gp.wr = reinterpret_cast<const bf16_t*>(a.w_router); gp.r1_given = a.r1_given;
    gp.x = a.x; gp.ids = a.ids; gp.gates = a.gates; gp.ids_out = a.ids_out;
    // k-splits: about one item per wave
    gp.ns = 1;
    while ((a.E / 16) * gp.ns * 2 <= kGateWaves && (a.d / 32) % (gp.ns * 2) == 0) gp.ns *= 2;
    const size_t glds = (2 * (size_t)a.d + 2 * (size_t)a.E * gp.ns) * sizeof(float);
    (void)hipGetLastError();
    const auto gate = a.E <= 64 ? moe_gate<1> : a.E <= 256 ? moe_gate<4> : moe_gate<kPerLane>;
    hipLaunchKernelGGL(gate, dim3(a.B), dim3(kGateThreads), glds, s, gp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ExpParams up;
    up.x = a.x;
    up.w = reinterpret_cast<const bf16_t*>(a.w_up);
    up.N = a.Fe; up.K = a.d; up.kk = kk; up.kp = a.k; up.nflows = a.nflows; up.ids = a.ids; up.kr = kr;
    up.P = a.B * kk;
    up.cpl_b = a.cpl_b; up.g_out = a.g_rows; up.y_out = nullptr; up.up = true;
    e = launch_expert<2>(up, a.E, s);
    if (e != hipSuccess) return e;
    ExpParams dn = up;
    dn.x = a.g_rows;
    dn.w = reinterpret_cast<const bf16_t*>(a.w_down);
    dn.N = a.d; dn.K = a.Fe; dn.g_out = nullptr; dn.y_out = a.y_rows; dn.up = false;
    e = launch_expert<2>(dn, a.E, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_combine, dim3(a.B), dim3(comb_threads(a.d)), 0, s, a.y_rows, a.gates, a.cpl_c, a.d, a.k,
                       ka, kr, kk, a.nflows, a.h, a.g_next, a.eps, a.x_next);
    return hipGetLastError();
}

}  // namespace dfk
