// Stacked-row skinny GEMM of the grouped decode step.
//
// Both flows of every sequence go through the same weight matrix together
// (gist.science/es/paper/2608.12385, "Arquitectura Central": all attention,
// MLP and output matrices are shared; "Costes de Inferencia vs.
// Entrenamiento": the two flows are grouped so the set of weights read does
// not grow), so each weight byte is read from HBM once per step:
// Y[m][n] = sum_k X[m][k] W[n][k] over the M = 2B stacked rows
// (row 2b = primary, 2b+1 = aux of sequence b).
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with the weights as the A operand,
// read from the 16x32 fragment layout (mfma_tile.h), the activation rows as
// the B operand from LDS; split over k-slices, persistent over row tiles;
// partial sums are finished by a reduce kernel with one of the epilogues:
// plain store, Q coupling + K/V append, GELU + b coupling, or c coupling +
// residual add (then LayerNorm), or left for the next kernel (EPI_PART). For
// matrices of 32M weights or more (16M with 4096 rows and columns or more)
// and up to 32 stacked rows, the activation
// fragments sit in registers instead (shape R: the waves of a workgroup split
// its k-slice and add their products through LDS). fp32 path (fp32 storage,
// row-major): one wave per weight row, lanes split K, wave reduction, same
// epilogues.
#include <algorithm>
#include <numeric>

#include "df_device.h"
#include "df_internal.h"
#include "mfma_tile.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

using tile::f32x4;

constexpr int kCUs = 256;   // compute units of the MI355X

struct GParams {
    const void* x;
    const void* w;
    int N, K;
    int M;          // logical rows: 2B (dual) or B (primary only)
    int row_step;   // physical stacked row of logical row m is m * row_step
    int nflows, B;
    int epi;
    float* out_f32;
    float* h;
    float* stats_out;
    float* x_out;
    const float* cpl;
    float* q_out;
    void* kc;
    void* vc;
    const int32_t* len;
    int H, Dh, S_max;
    int32_t* status;
    int S;                // k-slices
    float* part;          // split-K partials [S][M][N]
    const float* x_stats; // activation rows normalised on the fly (see GemvArgs)
    const float* x_gain;
    float eps;
    int halves;           // 2: the stacked rows are split over two workgroups of 64 (see gemv_bf16)
};

__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// Epilogue for weight row n of sequence b (y1 primary, y2 aux; y2 unused
// when only the primary flow runs). Rows in memory are stacked: 2b + f.
template <typename T>
__device__ __forceinline__ void epilogue(const GParams& p, int n, int b, float y1, float y2) {
    const bool dual = p.nflows == 2;
    const size_t r1 = (size_t)(2 * b) * p.N + n, r2 = r1 + p.N;
    switch (p.epi) {
        case EPI_STORE:
            p.out_f32[r1] = y1;
            if (dual) p.out_f32[r2] = y2;
            break;
        case EPI_GELU_B: {
            const float cb = (dual && p.cpl) ? p.cpl[n] : 0.f;   // loaded before any store
            const float g1 = gelu(y1);
            p.x_out[r1] = g1;
            if (dual) {
                float g2 = gelu(y2);
                if (p.cpl) g2 = fmaf(cb, g1, g2);                 // MLP-intermediate coupling (b_l)
                p.x_out[r2] = g2;
            }
            break;
        }
        case EPI_QKV: {
            const int d = p.H * p.Dh;
            if (n < d) {
                const size_t q1 = (size_t)(2 * b) * d + n;
                const float ca = (dual && p.cpl) ? p.cpl[n] : 0.f;   // loaded before the first store
                p.q_out[q1] = y1;
                if (dual) p.q_out[q1 + d] = p.cpl ? fmaf(ca, y1, y2) : y2;   // Q2 = Q2raw + a*Q1
            } else {
                // primary K/V only; the aux row's K/V part is discarded
                const int kvsel = (n - d) / d;
                const int nn = n - d - kvsel * d;
                const int hh = nn / p.Dh, i = nn - hh * p.Dh;
                const int pos = p.len[b];
                if (pos >= 0 && pos < p.S_max) {
                    T* cache = reinterpret_cast<T*>(kvsel == 0 ? p.kc : p.vc);
                    df::St<T>::st(cache, (((size_t)b * p.H + hh) * p.S_max + pos) * p.Dh + i, y1);
                } else if (p.status) {
                    p.status[0] |= 1;
                }
            }
            break;
        }
    }
}

typedef tile::u32x4 u32x4;
typedef tile::bf16x8 bf16x8;

// Epilogue from MFMA registers: lane l holds D[4*(l/16) + r][l%16] of its
// wave's 16 weight rows x 16 stacked rows (per m tile). With both flows, the
// aux row 2b+1 sits in the neighbouring lane of the primary row 2b.
template <int MT>
__device__ __forceinline__ void epilogue_regs(const GParams& p, const f32x4 (&acc)[MT], int n_base, int lane,
                                              int m0) {
    const int li = lane & 15, lg = lane >> 4;
    const bool dual = p.nflows == 2;
    #pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        #pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = acc[mt][r];
            const float partner = __shfl_xor(v, 1, 64);
            const int n = n_base + 4 * lg + r;
            const int m = m0 + mt * 16 + li;
            if (n >= p.N || m >= p.M) continue;
            if (dual) {
                if ((m & 1) == 0) epilogue<bf16_t>(p, n, m >> 1, v, partner);
            } else {
                epilogue<bf16_t>(p, n, m, v, 0.f);
            }
        }
    }
}

// Y = X W^T over one k-slice of KS columns, persistent over row tiles.
//
// Workgroup g works on slice s = g % S for a contiguous range of row tiles
// (16*RT weight rows each); its waves take the tiles of that range in turn.
// The activation slice is staged once per workgroup: each fp32 value is
// split into bf16 hi = rne(x) and lo = rne(x - hi) (x - hi - lo is below
// 2^-17 |x|) and both parts go through the matrix cores into the same fp32
// accumulator. Weights are read in the 16x32 fragment layout, so every
// wave-wide load is one contiguous 1 KiB piece, and a wave's tile slice is
// one contiguous run; the next NBUF - 1 batches of KU fragments per tile
// are always in flight (from before the activation staging on, and across
// tile boundaries). Loads are issued without branches (an
// iteration past the end reads a fixed hot address) so the compiler's wait
// counts stay exact. With S > 1 each tile's partial sums go to
// part[s][m][n] and a reduce kernel finishes in slice order; with S == 1
// the epilogue runs from the registers. EPI_PART always leaves the partial
// sums for the consumer to finish (the Q/K/V projection, which the
// attention pass finishes).
template <int MT, int RT, int KU, int NW, int KS, int NBUF>
__global__ __launch_bounds__(NW * 64) void gemv_bf16(GParams p) {
    extern __shared__ bf16_t xs[];
    constexpr int TR = 16 * RT, XS = KS + 8, IPT = KS / (32 * KU);
    constexpr int C4 = KS / 4, NI = 16 * MT * C4, XB = (NI + NW * 64 - 1) / (NW * 64);
    static_assert(KS % (32 * KU) == 0, "k-slice");
    static_assert(XB <= 16, "activation staging registers");
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int S = p.S;
    // With two row halves, workgroups b and b + 8 (dispatched together, on
    // the same XCD) take rows 0-63 and 64-127 of the same row tiles and
    // k-slice, so the second reads the weights from L2.
    const int item = p.halves == 2 ? (int)(((blockIdx.x >> 4) << 3) | (blockIdx.x & 7)) : (int)blockIdx.x;
    const int m0 = p.halves == 2 ? (int)((blockIdx.x >> 3) & 1) * 16 * MT : 0;
    const int s = item % S, grp = item / S, ngrp = gridDim.x / p.halves / S;
    const int n_tiles = (p.N + TR - 1) / TR;
    const int t_lo = (int)((long)grp * n_tiles / ngrp), t_hi = (int)((long)(grp + 1) * n_tiles / ngrp);
    const int my_tiles = t_hi - t_lo > wv ? (t_hi - t_lo - wv + NW - 1) / NW : 0;
    const int n_it = my_tiles * IPT;
    const int ks0 = s * KS, KB = p.K / 32, NT16 = p.N / 16;
    const bf16_t* W = reinterpret_cast<const bf16_t*>(p.w);
    const float* X = reinterpret_cast<const float*>(p.x);
    const bf16_t* dummy = reinterpret_cast<const bf16_t*>(X);
    bf16_t* xh = xs;
    bf16_t* xl = xs + 16 * MT * XS;

    auto load = [&](int it, u32x4 (&a)[RT][KU]) {
        const bool real = it < n_it;
        const int j = it / IPT, kb = it - j * IPT;
        const int tile = t_lo + wv + j * NW;
        #pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int t16 = min(tile * RT + rt, NT16 - 1);
            const bf16_t* q = W + (((size_t)t16 * KB + ks0 / 32 + kb * KU) * 64 + lane) * 8;
            q = real ? q : dummy;
            #pragma unroll
            for (int ku = 0; ku < KU; ++ku)
                a[rt][ku] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + (real ? 512 * ku : 0)));
        }
    };

    // Loads first: with a LayerNorm on the fly the gains of the slice and the
    // per-segment statistics of the rows (so the row statistics can be
    // combined while the rest is in flight), then the activation rows, then
    // the first weight fragments; then the normalisation and the hi/lo split.
    __shared__ float s_gain[KS];
    __shared__ float s_mean[16 * MT], s_rstd[16 * MT];
    // statistics: 16 lanes per row, lane j holds segment j (kMaxSeg == 16)
    constexpr int SPT = (16 * MT * kMaxSeg + NW * 64 - 1) / (NW * 64);
    static_assert(kMaxSeg == 16, "one 16-lane group per row");
    const bool norm = p.x_stats != nullptr;
    const int nseg = stat_segs(p.K);
    float4 gv = make_float4(0.f, 0.f, 0.f, 0.f);
    float2 sv[SPT];
    if (norm) {
        if ((int)threadIdx.x < KS / 4) gv = *reinterpret_cast<const float4*>(p.x_gain + ks0 + 4 * threadIdx.x);
        #pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int e = threadIdx.x + u * NW * 64;
            const int m = min(m0 + (e >> 4), p.M - 1), j = min(e & 15, nseg - 1);
            sv[u] = *reinterpret_cast<const float2*>(p.x_stats + ((size_t)(m * p.row_step) * nseg + j) * 2);
        }
    }
    float4 xv[XB];
    #pragma unroll
    for (int u = 0; u < XB; ++u) {
        const int i = min((int)threadIdx.x + u * NW * 64, NI - 1);
        const int m = i / C4, c = i - m * C4;
        xv[u] = *reinterpret_cast<const float4*>(X + (size_t)(min(m0 + m, p.M - 1) * p.row_step) * p.K + ks0 + c * 4);
    }
    static_assert(NBUF == 2 || NBUF == 3, "fragment buffers");
    u32x4 a0[RT][KU], a1[RT][KU], a2[NBUF == 3 ? RT : 1][NBUF == 3 ? KU : 1];
    load(0, a0);
    if constexpr (NBUF == 3) load(1, a1);
    if (norm) {
        // row mean and rstd by Chan's combination of the segments' (mean, M2),
        // reduced over each 16-lane group
        if ((int)threadIdx.x < KS / 4) *reinterpret_cast<float4*>(s_gain + 4 * threadIdx.x) = gv;
        #pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int e = threadIdx.x + u * NW * 64;
            const int m = e >> 4, j = e & 15;
            const bool valid = j < nseg;
            const float cnt = valid ? (float)min(kStatSeg, p.K - j * kStatSeg) : 0.f;
            const float mean = df::group_sum<16>(cnt * sv[u].x) / (float)p.K;
            const float dm = sv[u].x - mean;
            const float m2 = df::group_sum<16>(valid ? fmaf(cnt * dm, dm, sv[u].y) : 0.f);
            if (j == 0 && m < 16 * MT) {
                s_mean[m] = mean;
                s_rstd[m] = 1.0f / sqrtf(m2 / (float)p.K + p.eps);
            }
        }
        __syncthreads();
    }
    #pragma unroll
    for (int u = 0; u < XB; ++u) {
        const int i = threadIdx.x + u * NW * 64;
        if (i >= NI) break;
        const int m = i / C4, c = i - m * C4;
        float4 v = xv[u];
        if (norm) {
            const float mean = s_mean[m], rstd = s_rstd[m];
            const float4 g = *reinterpret_cast<const float4*>(s_gain + 4 * c);
            v.x = (v.x - mean) * rstd * g.x;
            v.y = (v.y - mean) * rstd * g.y;
            v.z = (v.z - mean) * rstd * g.z;
            v.w = (v.w - mean) * rstd * g.w;
        }
        uint2 hv, lv;
        df::split_hi_lo(v, hv, lv);
        *reinterpret_cast<uint2*>(xh + m * XS + c * 4) = hv;
        *reinterpret_cast<uint2*>(xl + m * XS + c * 4) = lv;
    }
    __syncthreads();

    f32x4 acc[RT][MT];
    #pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        #pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int xo = li * XS + lg * 8;

    // NBUF fragment buffers in rotation: NBUF - 1 batches are in flight while
    // one is consumed
    auto step = [&](int it, u32x4 (&cur)[RT][KU], u32x4 (&nxt)[RT][KU]) {
        load(it + NBUF - 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
        const int j = it / IPT, kb = it - j * IPT;
        const int kk = kb * 32 * KU;
        #pragma unroll
        for (int ku = 0; ku < KU; ++ku) {
            bf16x8 bh[MT], bl[MT];
            #pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int o = xo + mt * 16 * XS + kk + 32 * ku;
                bh[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xh + o));
                bl[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + o));
            }
            #pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, cur[rt][ku]);
                #pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh[mt], acc[rt][mt], 0, 0, 0);
                    acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl[mt], acc[rt][mt], 0, 0, 0);
                }
            }
        }
        if (kb == IPT - 1) {   // tile done
            const int tile = t_lo + wv + j * NW;
            #pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int nb = tile * TR + rt * 16;
                if (S > 1 || p.epi == EPI_RESID || p.epi == EPI_PART) {
                    #pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int m = m0 + mt * 16 + li, n0 = nb + 4 * lg;
                        if (n0 < p.N && m < p.M)
                            *reinterpret_cast<f32x4*>(p.part + ((size_t)s * p.M + m) * p.N + n0) = acc[rt][mt];
                    }
                } else {
                    epilogue_regs<MT>(p, acc[rt], nb, lane, m0);
                }
                #pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    int it = 0;
    if constexpr (NBUF == 3) {
        for (; it + 2 < n_it; it += 3) {
            step(it, a0, a2);
            step(it + 1, a1, a0);
            step(it + 2, a2, a1);
        }
        if (it < n_it) step(it, a0, a2);
        if (it + 1 < n_it) step(it + 1, a1, a0);
    } else {
        for (; it + 1 < n_it; it += 2) {
            step(it, a0, a1);
            step(it + 1, a1, a0);
        }
        if (it < n_it) step(it, a0, a1);
    }
}

// LayerNorm of the activation rows on the fly: the row mean and rstd come
// from the per-segment (mean, M2) of the residual reduce by Chan's
// combination, 16 lanes per row (lane j holds segment j), reduced by DPP
// sums. Loading (into registers) and reducing are separate steps, so the
// loads can be issued ahead of the weight stream and reduced after it.
template <int SPT, int NT>
struct RowStats {
    float2 sv[SPT];
    __device__ __forceinline__ void load(const GParams& p, int rows) {
        const int nseg = stat_segs(p.K);
        #pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int e = threadIdx.x + u * NT;
            const int m = min(min(e >> 4, rows - 1), p.M - 1), j = min(e & 15, nseg - 1);
            sv[u] = *reinterpret_cast<const float2*>(p.x_stats + ((size_t)(m * p.row_step) * nseg + j) * 2);
        }
    }
    __device__ __forceinline__ void reduce(const GParams& p, int rows, float* s_mean, float* s_rstd) const {
        const int nseg = stat_segs(p.K);
        #pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int e = threadIdx.x + u * NT;
            const int m = e >> 4, j = e & 15;
            const bool valid = j < nseg;
            const float cnt = valid ? (float)min(kStatSeg, p.K - j * kStatSeg) : 0.f;
            const float mean = df::group_sum<16>(cnt * sv[u].x) / (float)p.K;
            const float dm = sv[u].x - mean;
            const float m2 = df::group_sum<16>(valid ? fmaf(cnt * dm, dm, sv[u].y) : 0.f);
            if (j == 0 && m < rows) {
                s_mean[m] = mean;
                s_rstd[m] = 1.0f / sqrtf(m2 / (float)p.K + p.eps);
            }
        }
    }
};

// Activation fragment (B operand) of one 32-column block for one row: the
// lane's eight columns k0 .. k0 + 7 of row m, normalised when norm (gain g),
// split into bf16 hi and lo parts.
__device__ __forceinline__ void act_fragment(const float4& v0, const float4& v1, const float4& g0, const float4& g1,
                                             bool norm, float mean, float rstd, bf16x8& hi, bf16x8& lo) {
    float4 a = v0, b = v1;
    if (norm) {
        a = make_float4((a.x - mean) * rstd * g0.x, (a.y - mean) * rstd * g0.y, (a.z - mean) * rstd * g0.z,
                        (a.w - mean) * rstd * g0.w);
        b = make_float4((b.x - mean) * rstd * g1.x, (b.y - mean) * rstd * g1.y, (b.z - mean) * rstd * g1.z,
                        (b.w - mean) * rstd * g1.w);
    }
    uint2 h0, l0, h1, l1;
    df::split_hi_lo(a, h0, l0);
    df::split_hi_lo(b, h1, l1);
    hi = __builtin_bit_cast(bf16x8, (u32x4){h0.x, h0.y, h1.x, h1.y});
    lo = __builtin_bit_cast(bf16x8, (u32x4){l0.x, l0.y, l1.x, l1.y});
}

// Finished products of weight rows n0 .. n0 + 3 (y) for logical row m: the
// slice's partial sums, or with one slice the epilogue (the aux row 2b + 1
// is the neighbouring lane of the primary row 2b). Every lane of the wave
// calls it (the shuffle).
__device__ __forceinline__ void tile_out(const GParams& p, int s, int m, int n0, bool valid, const f32x4& y) {
    if (p.S > 1 || p.epi == EPI_RESID || p.epi == EPI_PART) {
        if (valid && m < p.M) *reinterpret_cast<f32x4*>(p.part + ((size_t)s * p.M + m) * p.N + n0) = y;
        return;
    }
    const bool dual = p.nflows == 2;
    #pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float partner = __shfl_xor(y[r], 1, 64);
        if (!valid || m >= p.M) continue;
        if (dual) {
            if ((m & 1) == 0) epilogue<bf16_t>(p, n0 + r, m >> 1, y[r], partner);
        } else {
            epilogue<bf16_t>(p, n0 + r, m, y[r], 0.f);
        }
    }
}

// Shape R (up to 32 stacked rows). The NW waves of a workgroup split its
// k-slice (KS = NW * KWB * 32 columns) into sub-ranges of KWB 32-column
// blocks; each wave holds the activation fragments of its sub-range in
// registers (hi and lo parts, normalised on the fly for a residual input)
// and streams the matching weight fragments of TB 16-row tiles per batch
// straight from global memory (one contiguous KWB KiB piece per tile), two
// batches in flight. The NW partial products of a batch are added in wave
// order through LDS (double-buffered) and stored as the slice's partial sums
// (or, with one slice, run through the epilogue). No activation fragment is
// read from LDS, and every wave of a workgroup does the same work.
template <int MT, int NW, int KWB, int TB>
__global__ __launch_bounds__(NW * 64) void gemv_r(GParams p) {
    constexpr int KS = NW * KWB * 32, NT = NW * 64, NP = TB * MT;
    constexpr int SPT = (16 * MT * 16 + NT - 1) / NT;
    extern __shared__ f32x4 red[];   // [2][NW][NP][64]
    __shared__ float s_mean[16 * MT], s_rstd[16 * MT];
    __shared__ float4 s_gain[NW][KWB * 8];   // each wave's gains, loaded once
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int S = p.S;
    const int s = blockIdx.x % S, grp = blockIdx.x / S, ngrp = gridDim.x / S;
    const int NT16 = p.N / 16, KB = p.K / 32;
    const int t_lo = (int)((long)grp * NT16 / ngrp), t_hi = (int)((long)(grp + 1) * NT16 / ngrp);
    const int nb = (t_hi - t_lo + TB - 1) / TB;
    const int kb0 = s * (KS / 32) + wv * KWB;
    const bf16_t* W = reinterpret_cast<const bf16_t*>(p.w);
    const float* X = reinterpret_cast<const float*>(p.x);
    const bool norm = p.x_stats != nullptr;

    // loads first: row statistics, the wave's gains (one float4 per lane
    // for the first KWB * 8 lanes; every lane group needs them, so they go
    // through LDS rather than being loaded 16 times), activations, then two
    // weight batches
    RowStats<SPT, NT> st;
    if (norm) st.load(p, 16 * MT);
    float4 g_own = make_float4(0.f, 0.f, 0.f, 0.f);
    if (norm && lane < KWB * 8) g_own = *reinterpret_cast<const float4*>(p.x_gain + kb0 * 32 + 4 * lane);
    float4 gv[KWB][2], xv[MT][KWB][2];
    #pragma unroll
    for (int kb = 0; kb < KWB; ++kb) {
        const int k = (kb0 + kb) * 32 + lg * 8;
        #pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = min(mt * 16 + li, p.M - 1);
            const float* q = X + (size_t)(m * p.row_step) * p.K + k;
            xv[mt][kb][0] = *reinterpret_cast<const float4*>(q);
            xv[mt][kb][1] = *reinterpret_cast<const float4*>(q + 4);
        }
    }
    const bf16_t* dummy = reinterpret_cast<const bf16_t*>(X);
    auto load = [&](int j, u32x4 (&a)[TB][KWB]) {
        #pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = t_lo + j * TB + tb;
            const bool real = j < nb && t < t_hi;
            const bf16_t* q = W + (((size_t)min(t, NT16 - 1) * KB + kb0) * 64 + lane) * 8;
            q = real ? q : dummy;   // past the end: a fixed hot address, no branch
            #pragma unroll
            for (int kb = 0; kb < KWB; ++kb)
                a[tb][kb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q + (real ? 512 * kb : 0)));
        }
    };
    u32x4 a0[TB][KWB], a1[TB][KWB];
    load(0, a0);
    load(1, a1);
    if (norm) {
        if (lane < KWB * 8) s_gain[wv][lane] = g_own;
        st.reduce(p, 16 * MT, s_mean, s_rstd);
        __syncthreads();
        #pragma unroll
        for (int kb = 0; kb < KWB; ++kb) {
            gv[kb][0] = s_gain[wv][kb * 8 + lg * 2];
            gv[kb][1] = s_gain[wv][kb * 8 + lg * 2 + 1];
        }
    }
    bf16x8 xh[MT][KWB], xl[MT][KWB];
    #pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + li;
        const float mean = norm ? s_mean[m] : 0.f, rstd = norm ? s_rstd[m] : 0.f;
        #pragma unroll
        for (int kb = 0; kb < KWB; ++kb)
            act_fragment(xv[mt][kb][0], xv[mt][kb][1], gv[kb][0], gv[kb][1], norm, mean, rstd, xh[mt][kb],
                         xl[mt][kb]);
    }

    auto step = [&](int j, u32x4 (&cur)[TB][KWB]) {
        f32x4 acc[TB][MT];
        #pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            #pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[tb][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        #pragma unroll
        for (int kb = 0; kb < KWB; ++kb)
            #pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, cur[tb][kb]);
                #pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[tb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, xh[mt][kb], acc[tb][mt], 0, 0, 0);
                    acc[tb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, xl[mt][kb], acc[tb][mt], 0, 0, 0);
                }
            }
        load(j + 2, cur);
        f32x4* rb = red + (size_t)(j & 1) * NW * NP * 64;
        #pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            #pragma unroll
            for (int mt = 0; mt < MT; ++mt) rb[((size_t)wv * NP + tb * MT + mt) * 64 + lane] = acc[tb][mt];
        __syncthreads();
        for (int pr = wv; pr < NP; pr += NW) {   // waves add the NW partial products in wave order
            const int tb = pr / MT, mt = pr - (pr / MT) * MT;
            f32x4 y = rb[(size_t)pr * 64 + lane];
            #pragma unroll
            for (int w = 1; w < NW; ++w) y += rb[((size_t)w * NP + pr) * 64 + lane];
            const int t = t_lo + j * TB + tb;
            tile_out(p, s, mt * 16 + li, t * 16 + 4 * lg, t < t_hi, y);
        }
    };
    int j = 0;
    for (; j + 1 < nb; j += 2) {
        step(j, a0);
        step(j + 1, a1);
    }
    if (j < nb) step(j, a0);
}

// Sums of the S k-slice partials of logical rows m1 and m2 (m2 < 0: none),
// column n, in slice order; the loads of SB slices (2 SB values) are in
// flight together.
template <int SB>
__device__ __forceinline__ void sum_slices_sb(const GParams& p, int S, int m1, int m2, int n, float& y1, float& y2) {
    const float* q1 = p.part + (size_t)m1 * p.N + n;
    const float* q2 = p.part + (size_t)(m2 < 0 ? m1 : m2) * p.N + n;
    const size_t stride = (size_t)p.M * p.N;
    float v1 = 0.f, v2 = 0.f;
    for (int s = 0; s < S; s += SB) {
        float t1[SB], t2[SB];
        #pragma unroll
        for (int u = 0; u < SB; ++u) {
            const size_t o = (size_t)min(s + u, S - 1) * stride;
            t1[u] = q1[o];
            t2[u] = q2[o];
        }
        #pragma unroll
        for (int u = 0; u < SB; ++u) {
            if (s + u >= S) break;
            v1 += t1[u];
            v2 += t2[u];
        }
    }
    y1 = v1;
    y2 = m2 < 0 ? 0.f : v2;
}

// The batch is sized to S (uniform branch), so no load is spent on a clamped
// slice when S <= 4 or 8; the sums are the same either way.
__device__ __forceinline__ void sum_slices(const GParams& p, int S, int m1, int m2, int n, float& y1, float& y2) {
    if (S <= 4) sum_slices_sb<4>(p, S, m1, m2, n, y1, y2);
    else if (S <= 8) sum_slices_sb<8>(p, S, m1, m2, n, y1, y2);
    else sum_slices_sb<16>(p, S, m1, m2, n, y1, y2);
}

// Split-K finish for the elementwise epilogues: thread per (sequence, column).
__global__ __launch_bounds__(256) void gemv_reduce_epi(GParams p, int S) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = t / p.N, n = t - (t / p.N) * p.N;
    if (b >= p.B) return;
    const bool dual = p.nflows == 2;
    float y1, y2;
    sum_slices(p, S, dual ? 2 * b : b, dual ? 2 * b + 1 : -1, n, y1, y2);
    epilogue<bf16_t>(p, n, b, y1, y2);
}

// Split-K finish with the residual add: block (segment, sequence), thread
// per column; the aux output gets the c coupling (y2 += c * y1) when given;
// h += y; then the (mean, M2) of each updated row over the block's
// kStatSeg columns go to stats_out, from which the next projection (or
// ln_apply) normalises the rows without another pass.
__global__ __launch_bounds__(kStatSeg) void gemv_reduce_resid(GParams p, int S) {
    __shared__ float2 red[kStatSeg / 64];
    const int seg = blockIdx.x, b = blockIdx.y, nseg = gridDim.x;
    const int n = seg * kStatSeg + threadIdx.x;
    const bool ok = n < p.N;
    const bool dual = p.nflows == 2;
    float v1 = 0.f, v2 = 0.f;
    if (ok) {
        // every load (residual rows, coupling) before the first store, so
        // they are in flight with the partial sums
        float* h1 = p.h + (size_t)(2 * b) * p.N + n;
        float* h2 = p.h + (size_t)(2 * b + 1) * p.N + n;
        const float h1v = *h1;
        const float h2v = dual ? *h2 : 0.f;
        const float cc = (dual && p.cpl) ? p.cpl[n] : 0.f;
        float y1, y2;
        sum_slices(p, S, dual ? 2 * b : b, dual ? 2 * b + 1 : -1, n, y1, y2);
        v1 = h1v + y1;
        *h1 = v1;
        if (dual) {
            if (p.cpl) y2 = fmaf(cc, y1, y2);   // MLP-output coupling (c_l)
            v2 = h2v + y2;
            *h2 = v2;
        }
    }
    if (!p.stats_out) return;
    // both rows at once: block sums of (v1, v2), then of the squared deviations
    auto bsum2 = [&](float a, float c) {
        a = df::wave_sum(a);
        c = df::wave_sum(c);
        __syncthreads();
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(a, c);
        __syncthreads();
        float2 t = red[0];
        #pragma unroll
        for (int i = 1; i < kStatSeg / 64; ++i) { t.x += red[i].x; t.y += red[i].y; }
        return t;
    };
    const float cnt = (float)min(kStatSeg, p.N - seg * kStatSeg);
    const float2 sm = bsum2(v1, v2);
    const float mean1 = sm.x / cnt, mean2 = sm.y / cnt;
    const float d1 = ok ? v1 - mean1 : 0.f, d2 = ok ? v2 - mean2 : 0.f;
    const float2 m2 = bsum2(d1 * d1, d2 * d2);
    if (threadIdx.x == 0) {
        float* st = p.stats_out + ((size_t)(2 * b) * nseg + seg) * 2;
        st[0] = mean1;
        st[1] = m2.x;
        if (dual) {
            st[(size_t)nseg * 2] = mean2;
            st[(size_t)nseg * 2 + 1] = m2.y;
        }
    }
}

// fp32 storage: one wave per weight row, all stacked rows at once (M <= 16).
__global__ __launch_bounds__(256) void gemv_f32(GParams p) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= p.N) return;
    const float* W = reinterpret_cast<const float*>(p.w) + (size_t)n * p.K;
    const float* X = reinterpret_cast<const float*>(p.x);
    float acc[16];
    #pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] = 0.f;
    for (int k = lane * 4; k < p.K; k += 256) {
        const float4 wv = *reinterpret_cast<const float4*>(W + k);
        #pragma unroll
        for (int m = 0; m < 16; ++m) {
            if (m < p.M) {
                const float4 xv = *reinterpret_cast<const float4*>(X + (size_t)(m * p.row_step) * p.K + k);
                acc[m] = fmaf(wv.x, xv.x, acc[m]);
                acc[m] = fmaf(wv.y, xv.y, acc[m]);
                acc[m] = fmaf(wv.z, xv.z, acc[m]);
                acc[m] = fmaf(wv.w, xv.w, acc[m]);
            }
        }
    }
    #pragma unroll
    for (int m = 0; m < 16; ++m)
        if (m < p.M) acc[m] = df::wave_sum(acc[m]);
    if (p.epi == EPI_RESID) {          // one "slice"; gemv_reduce_resid finishes
        #pragma unroll
        for (int m = 0; m < 16; ++m)
            if (m < p.M && lane == m) p.part[(size_t)m * p.N + n] = acc[m];
        return;
    }
    const bool dual = p.nflows == 2;
    #pragma unroll
    for (int b = 0; b < 8; ++b) {
        if (b < p.B && lane == b) {
            const float y1 = dual ? acc[2 * b] : acc[b];
            const float y2 = dual ? acc[2 * b + 1] : 0.f;
            epilogue<float>(p, n, b, y1, y2);
        }
    }
}

// Kernel shapes: A = 16-row tiles, 8 waves (12 with 64 stacked rows), batches
// of 8 fragments (4 with 64 stacked rows, 2 with 128), two batches ahead (one
// with 128 rows);
// B = 32-row tiles, 4 waves, batches of 4 fragments per tile, one batch ahead
// (up to 32 stacked rows, for matrices with fewer than 8192 rows or at most
// 16 M weights; plan_gemv holds the choice).
// R: the register-resident shape above (gemv_r, up to 32 stacked rows).
enum Variant { VAR_A = 0, VAR_B = 1, VAR_R = 2 };

template <typename K>
hipError_t launch_kernel(K* fn, GParams& p, const GemvPlan& pl, int threads, hipStream_t s) {
    hipError_t e = tile::allow_lds(reinterpret_cast<const void*>(fn), pl.lds);
    if (e != hipSuccess) return e;
    (void)hipGetLastError();
    hipLaunchKernelGGL(fn, dim3(pl.grid), dim3(threads), pl.lds, s, p);
    return hipGetLastError();
}

hipError_t launch_r(GParams& p, const GemvPlan& pl, hipStream_t s) {
    if (pl.MT == 1) return launch_kernel(&gemv_r<1, 8, 4, 2>, p, pl, 512, s);
    return launch_kernel(&gemv_r<2, 8, 4, 2>, p, pl, 512, s);
}

template <int MT, int RT, int KU, int NW, int KS, int NBUF>
hipError_t launch_one(GParams& p, const GemvPlan& pl, hipStream_t s) {
    const void* fn = reinterpret_cast<const void*>(&gemv_bf16<MT, RT, KU, NW, KS, NBUF>);
    hipError_t e = tile::allow_lds(fn, pl.lds);
    if (e != hipSuccess) return e;
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemv_bf16<MT, RT, KU, NW, KS, NBUF>), dim3(pl.grid), dim3(NW * 64), pl.lds, s, p);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(GParams& p, const GemvPlan& pl, hipStream_t s) {
    if (pl.variant == VAR_B) {
        if constexpr (MT <= 2) {
            if (pl.ks == 512) return launch_one<MT, 2, 4, 4, 512, 2>(p, pl, s);
            if (pl.ks == 256) return launch_one<MT, 2, 4, 4, 256, 2>(p, pl, s);
        }
        return hipErrorInvalidValue;
    }
    constexpr int KU = MT >= 8 ? 2 : MT >= 4 ? 4 : 8;   // register budget of the wider activation tiles
    constexpr int NB = MT >= 8 ? 2 : 3;
    if constexpr (MT <= 2) {
        if (pl.ks == 1024) return launch_one<MT, 1, KU, 8, 1024, NB>(p, pl, s);
        if (pl.ks == 512) return launch_one<MT, 1, KU, 8, 512, NB>(p, pl, s);
    }
    if constexpr (MT == 4) {
        // 12 waves (three per SIMD; 163 VGPRs): the MoE step's Q/K/V gives
        // each workgroup 12 row tiles, one per wave instead of two on half
        // of eight waves
        if (pl.ks == 512) return launch_one<MT, 1, KU, 12, 512, NB>(p, pl, s);
    }
    if (pl.ks == 256) return launch_one<MT, 1, KU, 8, 256, NB>(p, pl, s);
    return hipErrorInvalidValue;
}

hipError_t finish(GParams& p, int S, hipStream_t s) {
    if (p.epi == EPI_RESID) {
        hipLaunchKernelGGL(gemv_reduce_resid, dim3(stat_segs(p.N), p.B), dim3(kStatSeg), 0, s, p, S);
        return hipGetLastError();
    }
    if (S > 1 && p.epi != EPI_PART) {
        const long total = (long)p.B * p.N;
        hipLaunchKernelGGL(gemv_reduce_epi, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p, S);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

namespace {

// k-slice widths the kernel shapes are instantiated for (launch_mt).
bool ks_supported(int variant, int MT, int ks) {
    if (variant == VAR_B) return MT <= 2 && (ks == 512 || ks == 256);
    if (ks == 1024) return MT <= 2;
    if (ks == 512) return MT <= 4;
    return ks == 256;
}

// Widest supported k-slice for a shape (from a plan sweep on the box, weights
// rotated past the MALL): 256 for the smallest matrices in the 32-row-tile
// shape, else the widest the activation tile leaves LDS for.
int ks_for(int variant, int MT, int N, int K) {
    const long nk = (long)N * K;
    const int ks_max = variant == VAR_B ? (nk <= (4L << 20) ? 256 : 512) : (MT <= 2 ? 1024 : MT == 4 ? 512 : 256);
    for (int c = ks_max; c >= 256; c /= 2)
        if (K % c == 0) return c;
    return 256;
}

int variant_for(int MT, int N, int K) {
    // 32-row tiles up to 16M weights or below 8192 rows
    return (MT <= 2 && (N < 8192 || (long)N * K <= (16L << 20))) ? VAR_B : VAR_A;
}

int mt_for(int M) {
    const int mt = (M + 15) / 16;
    return mt <= 1 ? 1 : mt <= 2 ? 2 : mt <= 4 ? 4 : 8;
}

}  // namespace

GemvPlan plan_gemv(int dtype, int N, int K, int M, int M_slices) {
    GemvPlan pl{};
    pl.halves = 1;
    if (M_slices < M) M_slices = M;
    if (dtype != DF_BF16 || M < 1 || M_slices > 128 || N < 16 || N % 16 || K < 256 || K % 256) return pl;
    pl.MT = mt_for(M);
    // The shape and the k-slice width follow from the planned row count only,
    // so every output is summed over the same slices, in the same order,
    // whichever row count runs (a primary-only step gives bitwise the primary
    // results of a dual step). The register-resident shape where it measured
    // faster inside the decode step (per-kernel traces): up to 32 rows and
    // matrices of 32M weights or more, or of 16M with at least 4096 rows and
    // columns (1024-wide slices; the 1.3B model's 2048-row down projection
    // measured slower in it).
    const int mt_s = mt_for(M_slices);
    const int NT16 = N / 16;
    const long nk = (long)N * K;
    if (mt_s <= 2 && (nk >= (32L << 20) || (nk >= (16L << 20) && N >= 4096 && K >= 4096)) && K % 1024 == 0) {
        pl.variant = VAR_R;
        pl.ks = 1024;
        pl.lds = (size_t)2 * 8 * 2 * pl.MT * 64 * 16;   // the waves' partial products, double-buffered
        pl.S = K / pl.ks;
        const int ngrp = std::min(std::max(1, kCUs / pl.S), NT16);
        pl.grid = ngrp * pl.S;
        pl.part_floats = (size_t)pl.S * M * N;
        return pl;
    }
    // the k-slice width of the M_slices-row plan (the kernel shape may differ:
    // the k order within a slice is the same in both)
    int ks = ks_for(variant_for(mt_s, N, K), mt_s, N, K);
    if (mt_s == 8 && K % 512 == 0) {
        // 65-128 planned rows: 512-wide slices, the rows split into two
        // workgroups of 64 (a 128-row tile would leave LDS for 256 columns
        // only, and the split-K partials grow with the slice count)
        ks = 512;
        if (pl.MT == 8) {
            pl.MT = 4;
            pl.halves = 2;
        }
    }
    pl.variant = variant_for(pl.MT, N, K);
    if (!ks_supported(pl.variant, pl.MT, ks)) return GemvPlan{};
    pl.ks = ks;
    pl.S = K / ks;
    pl.lds = (size_t)2 * 16 * pl.MT * (ks + 8) * 2;
    // one or two resident workgroups per CU (LDS permitting), split over the
    // k-slices; no more row groups than row tiles
    const size_t lds_static = (size_t)ks * 4 + 2 * 16 * pl.MT * 4;   // gains, row mean and rstd
    const int wg_per_cu = pl.variant == VAR_A && pl.lds + lds_static <= 80 * 1024 ? 2 : 1;
    const int rt = pl.variant == VAR_B ? 2 : 1;
    const int n_tiles = (N + 16 * rt - 1) / (16 * rt);
    int ngrp = std::max(1, kCUs * wg_per_cu / (pl.S * pl.halves));
    ngrp = std::min(ngrp, n_tiles);
    if (pl.halves == 2) {
        // the pairing of workgroups b and b + 8 needs ngrp * S % 8 == 0
        // (groups past the last row tile have no tiles and exit)
        const int g = 8 / std::gcd(pl.S, 8);
        ngrp = std::max(g, ngrp / g * g);
    }
    pl.grid = ngrp * pl.S * pl.halves;
    pl.part_floats = (size_t)pl.S * M * N;   // used when S > 1 or before a residual + norm
    return pl;
}

hipError_t gemv(const GemvArgs& a, hipStream_t s) {
    GParams p;
    p.x = a.x; p.w = a.w; p.N = a.N; p.K = a.K; p.nflows = a.nflows; p.B = a.B;
    p.M = a.nflows == 2 ? 2 * a.B : a.B;
    p.row_step = a.nflows == 2 ? 1 : 2;
    p.epi = a.epi; p.out_f32 = a.out_f32; p.h = a.h; p.stats_out = a.stats_out; p.x_out = a.x_out; p.cpl = a.cpl;
    p.q_out = a.q_out; p.x_stats = a.x_stats; p.x_gain = a.x_gain;
    p.kc = a.kc; p.vc = a.vc; p.len = a.len; p.H = a.H; p.Dh = a.Dh; p.S_max = a.S_max; p.status = a.status;
    p.part = a.part; p.eps = a.eps;
    if (a.dtype == DF_F32) {
        if (p.M > 16 || a.epi == EPI_PART) return hipErrorInvalidValue;
        if (a.x_stats) return hipErrorInvalidValue;   // fp32 rows are normalised by ln_apply
        if (a.epi == EPI_RESID && (!a.part || a.N > 4096)) return hipErrorInvalidValue;
        (void)hipGetLastError();
        hipLaunchKernelGGL(gemv_f32, dim3((a.N + 3) / 4), dim3(256), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return finish(p, 1, s);
    }
    const GemvPlan pl = plan_gemv(a.dtype, a.N, a.K, p.M, a.slice_rows);
    if (pl.MT == 0) return hipErrorInvalidValue;
    p.S = pl.S;
    p.halves = pl.halves;
    if ((pl.S > 1 || a.epi == EPI_RESID || a.epi == EPI_PART) && !a.part) return hipErrorInvalidValue;
    if (a.epi == EPI_RESID && a.N > 4096) return hipErrorInvalidValue;
    if (a.x_stats && (!a.x_gain || a.K > kMaxSeg * kStatSeg)) return hipErrorInvalidValue;
    hipError_t e;
    if (pl.variant == VAR_R) {
        e = launch_r(p, pl, s);
        if (e != hipSuccess) return e;
        return finish(p, pl.S, s);
    }
    switch (pl.MT) {
        case 1: e = launch_mt<1>(p, pl, s); break;
        case 2: e = launch_mt<2>(p, pl, s); break;
        case 4: e = launch_mt<4>(p, pl, s); break;
        default: e = launch_mt<8>(p, pl, s); break;
    }
    if (e != hipSuccess) return e;
    return finish(p, pl.S, s);
}

}  // namespace dfk
