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
// bf16 path (v_mfma_f32_16x16x32_bf16): a workgroup owns 32 weight rows
// (two 16-row A tiles) and splits K across its waves; each lane streams
// 16-byte pieces of weight rows (A operand: row = lane%16, k-group =
// lane/16) and of activation rows (B operand: column = stacked row).
// The per-wave partial sums meet in LDS in a fixed order, then one fused
// epilogue per output element: plain store, Q coupling + K/V append, GELU +
// b coupling, or c coupling + residual add. fp32 path (fp32 storage): one
// wave per weight row, lanes split K, wave reduction, same epilogues.
#include <algorithm>

#include "df_device.h"
#include "df_internal.h"
#include "mfma_tile.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

using tile::f32x4;

struct GParams {
    const void* x;
    const void* w;
    int N, K;
    int M;          // logical rows: 2B (dual) or B (primary only)
    int row_step;   // physical stacked row of logical row m is m * row_step
    int nflows, B, kw;
    int epi;
    float* out_f32;
    float* h;
    float* x_out;
    const float* cpl;
    float* q_out;
    void* kc;
    void* vc;
    const int32_t* len;
    int H, Dh, S_max;
    int32_t* status;
    float* part;          // split-K partials [S][M][N]
    const float* ln_gain; // EPI_RESID_LN: gain of the norm that follows
    float eps;
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
            const float g1 = gelu(y1);
            p.x_out[r1] = g1;
            if (dual) {
                float g2 = gelu(y2);
                if (p.cpl) g2 = fmaf(p.cpl[n], g1, g2);          // MLP-intermediate coupling (b_l)
                p.x_out[r2] = g2;
            }
            break;
        }
        case EPI_QKV: {
            const int d = p.H * p.Dh;
            if (n < d) {
                const size_t q1 = (size_t)(2 * b) * d + n;
                p.q_out[q1] = y1;
                if (dual) p.q_out[q1 + d] = p.cpl ? fmaf(p.cpl[n], y1, y2) : y2;   // Q2 = Q2raw + a*Q1
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

constexpr int NWAVE = 8;         // waves per workgroup, 16 weight rows each
constexpr int WG_ROWS = 16 * NWAVE;

// Epilogue from MFMA registers: lane l holds D[4*(l/16) + r][l%16] of its
// wave's 16 rows x 16 stacked rows (per m tile). With both flows, the aux
// row 2b+1 sits in the neighbouring lane of the primary row 2b.
template <int MT>
__device__ __forceinline__ void epilogue_regs(const GParams& p, const f32x4 (&acc)[MT], int n_base, int lane) {
    const int li = lane & 15, lg = lane >> 4;
    const bool dual = p.nflows == 2;
    #pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        #pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = acc[mt][r];
            const float partner = __shfl_xor(v, 1, 64);
            const int n = n_base + 4 * lg + r;
            const int m = mt * 16 + li;
            if (n >= p.N || m >= p.M) continue;
            if (dual) {
                if ((m & 1) == 0) epilogue<bf16_t>(p, n, m >> 1, v, partner);
            } else {
                epilogue<bf16_t>(p, n, m, v, 0.f);
            }
        }
    }
}

// Y = X W^T for NWAVE*16 weight rows over one k-slice [s*ks, (s+1)*ks).
// Activation rows are fp32; while the k-slice is staged in LDS each value is
// split into bf16 hi = rne(x) and lo = rne(x - hi) (x - hi - lo is below
// 2^-17 |x|), and both parts go through the matrix cores into the same fp32
// accumulator. LDS rows are padded by 8 elements against bank conflicts and
// shared by the waves; each wave streams its 16 weight rows from HBM with the
// next KU chunks already in flight. With S = gridDim.y > 1 slices, every
// workgroup writes its partial sums and the last one to finish (atomic
// counter per row block) adds the S partials in slice order and runs the
// epilogue: deterministic, no float atomics.
template <int MT, int KU>
__global__ __launch_bounds__(NWAVE * 64) void gemv_bf16(GParams p) {
    extern __shared__ bf16_t xs[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int blk = blockIdx.x, sl = blockIdx.y, S = gridDim.y;
    const int n_base = blk * WG_ROWS + wv * 16;
    const int ks = p.kw, ks0 = sl * ks;
    const int XS = ks + 8;
    bf16_t* xs_hi = xs;
    bf16_t* xs_lo = xs + 16 * MT * XS;
    const int li = lane & 15, lg = lane >> 4;
    const bf16_t* W = reinterpret_cast<const bf16_t*>(p.w);
    const float* X = reinterpret_cast<const float*>(p.x);
    const bf16_t* wp = W + (size_t)min(n_base + li, p.N - 1) * p.K + ks0 + lg * 8;

    u32x4 a0[KU];
    #pragma unroll
    for (int ku = 0; ku < KU; ++ku) a0[ku] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + 32 * ku));

    // Stage the activation k-slice (loads of a batch issued before any is used).
    const int c4 = ks >> 2, n_items = 16 * MT * c4;
    constexpr int SB = 8;
    for (int i0 = threadIdx.x; i0 < n_items; i0 += SB * NWAVE * 64) {
        float4 v[SB];
        #pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int i = i0 + u * NWAVE * 64;
            if (i < n_items) {
                const int m = i / c4, c = i - m * c4;
                const int mm = min(m, p.M - 1);
                v[u] = *reinterpret_cast<const float4*>(X + (size_t)(mm * p.row_step) * p.K + ks0 + c * 4);
            }
        }
        #pragma unroll
        for (int u = 0; u < SB; ++u) {
            const int i = i0 + u * NWAVE * 64;
            if (i < n_items) {
                const int m = i / c4, c = i - m * c4;
                const bf16_t h0 = df::f32_to_bf16(v[u].x), h1 = df::f32_to_bf16(v[u].y);
                const bf16_t h2 = df::f32_to_bf16(v[u].z), h3 = df::f32_to_bf16(v[u].w);
                const bf16_t l0 = df::f32_to_bf16(v[u].x - df::bf16_to_f32(h0));
                const bf16_t l1 = df::f32_to_bf16(v[u].y - df::bf16_to_f32(h1));
                const bf16_t l2 = df::f32_to_bf16(v[u].z - df::bf16_to_f32(h2));
                const bf16_t l3 = df::f32_to_bf16(v[u].w - df::bf16_to_f32(h3));
                uint2 hv, lv;
                hv.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
                hv.y = (uint32_t)h2 | ((uint32_t)h3 << 16);
                lv.x = (uint32_t)l0 | ((uint32_t)l1 << 16);
                lv.y = (uint32_t)l2 | ((uint32_t)l3 << 16);
                *reinterpret_cast<uint2*>(xs_hi + m * XS + c * 4) = hv;
                *reinterpret_cast<uint2*>(xs_lo + m * XS + c * 4) = lv;
            }
        }
    }
    __syncthreads();

    f32x4 acc[MT];
    #pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int xoff = li * XS + lg * 8;
    for (int kk = 0; kk < ks; kk += 32 * KU) {
        const bool more = kk + 32 * KU < ks;
        u32x4 a1[KU];
        if (more) {
            #pragma unroll
            for (int ku = 0; ku < KU; ++ku)
                a1[ku] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + kk + 32 * KU + 32 * ku));
        }
        #pragma unroll
        for (int ku = 0; ku < KU; ++ku) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, a0[ku]);
            #pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int o = xoff + mt * 16 * XS + kk + 32 * ku;
                const u32x4 bh = *reinterpret_cast<const u32x4*>(xs_hi + o);
                const u32x4 bl = *reinterpret_cast<const u32x4*>(xs_lo + o);
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bh), acc[mt], 0, 0, 0);
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bl), acc[mt], 0, 0, 0);
            }
        }
        if (more) {
            #pragma unroll
            for (int ku = 0; ku < KU; ++ku) a0[ku] = a1[ku];
        }
    }

    if (S > 1 || p.epi == EPI_RESID_LN) {
        // partial sums of this k-slice: part[sl][m][n]; a reduce kernel finishes
        #pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = n_base + 4 * lg + r, m = mt * 16 + li;
                if (n < p.N && m < p.M) p.part[((size_t)sl * p.M + m) * p.N + n] = acc[mt][r];
            }
        return;
    }
    epilogue_regs<MT>(p, acc, n_base, lane);
}

// Sum of the S k-slice partials of logical row m, column n (slice order;
// loads issued eight at a time).
__device__ __forceinline__ float sum_slices(const GParams& p, int S, int m, int n) {
    const float* q = p.part + (size_t)m * p.N + n;
    const size_t stride = (size_t)p.M * p.N;
    float v = 0.f;
    int s = 0;
    for (; s + 8 <= S; s += 8) {
        float t[8];
        #pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = q[(size_t)(s + u) * stride];
        #pragma unroll
        for (int u = 0; u < 8; ++u) v += t[u];
    }
    for (; s < S; ++s) v += q[(size_t)s * stride];
    return v;
}

// Split-K finish for the elementwise epilogues: thread per (sequence, column).
__global__ __launch_bounds__(256) void gemv_reduce_epi(GParams p, int S) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = t / p.N, n = t - (t / p.N) * p.N;
    if (b >= p.B) return;
    const bool dual = p.nflows == 2;
    const float y1 = sum_slices(p, S, dual ? 2 * b : b, n);
    const float y2 = dual ? sum_slices(p, S, 2 * b + 1, n) : 0.f;
    epilogue<bf16_t>(p, n, b, y1, y2);
}

// Split-K finish with the residual add: thread per (sequence, column); the
// aux output gets the c coupling (y2 += c * y1) when given; h += y. The
// following LayerNorm runs as its own row kernel.
__global__ __launch_bounds__(256) void gemv_reduce_resid(GParams p, int S) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = t / p.N, n = t - (t / p.N) * p.N;
    if (b >= p.B) return;
    const bool dual = p.nflows == 2;
    const float y1 = sum_slices(p, S, dual ? 2 * b : b, n);
    p.h[(size_t)(2 * b) * p.N + n] += y1;
    if (dual) {
        float y2 = sum_slices(p, S, 2 * b + 1, n);
        if (p.cpl) y2 = fmaf(p.cpl[n], y1, y2);   // MLP-output coupling (c_l)
        p.h[(size_t)(2 * b + 1) * p.N + n] += y2;
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
    if (p.epi == EPI_RESID_LN) {       // one "slice"; gemv_reduce_ln finishes
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

template <int MT>
constexpr int ku_of() { return MT <= 2 ? 8 : (MT == 4 ? 4 : 2); }

template <int MT>
hipError_t launch_bf16(GParams& p, const GemvPlan& pl, hipStream_t s) {
    constexpr int KU = ku_of<MT>();
    p.kw = pl.ks;
    hipError_t e = tile::allow_lds(reinterpret_cast<const void*>(&gemv_bf16<MT, KU>), pl.lds);
    if (e != hipSuccess) return e;
    (void)hipGetLastError();
    hipLaunchKernelGGL((gemv_bf16<MT, KU>), dim3(pl.nblocks, pl.S), dim3(NWAVE * 64), pl.lds, s, p);
    return hipGetLastError();
}

hipError_t finish(GParams& p, int S, hipStream_t s) {
    if (p.epi == EPI_RESID_LN) {
        const long total = (long)p.B * p.N;
        hipLaunchKernelGGL(gemv_reduce_resid, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p, S);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return layer_norm_rows(DF_F32, p.h, p.ln_gain, p.eps, p.B, p.N, p.nflows, p.x_out, s);
    }
    if (S > 1) {
        const long total = (long)p.B * p.N;
        hipLaunchKernelGGL(gemv_reduce_epi, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p, S);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

GemvPlan plan_gemv(int dtype, int N, int K, int M) {
    GemvPlan pl{};
    if (dtype != DF_BF16) return pl;
    int mt = (M + 15) / 16;
    pl.MT = mt <= 1 ? 1 : mt <= 2 ? 2 : mt <= 4 ? 4 : 8;
    pl.nblocks = (N + WG_ROWS - 1) / WG_ROWS;
    // k-slice: a divisor of K, multiple of 32*KU, activation slice (hi and lo
    // parts) in LDS small enough for two workgroups per CU; smaller slices
    // until about two workgroups per CU are in the grid.
    const int KU = pl.MT <= 2 ? 8 : (pl.MT == 4 ? 4 : 2);
    const int step = 32 * KU;
    auto lds_of = [&](int ks) { return (size_t)2 * 16 * pl.MT * (ks + 8) * 2; };
    int best = step;
    for (int ks = step; ks <= K && ks <= 512; ks += step)
        if (K % ks == 0 && lds_of(ks) <= 78 * 1024) best = ks;
    int ks = best;
    while ((long)pl.nblocks * (K / ks) < 512) {
        int nxt = 0;
        for (int c = step; c < ks; c += step)
            if (K % c == 0) nxt = c;
        if (nxt == 0) break;
        ks = nxt;
    }
    pl.ks = ks;
    pl.S = K / ks;
    pl.lds = lds_of(ks);
    pl.part_floats = (size_t)pl.S * M * N;   // used when S > 1 or before a residual + norm
    return pl;
}

hipError_t gemv(const GemvArgs& a, hipStream_t s) {
    GParams p;
    p.x = a.x; p.w = a.w; p.N = a.N; p.K = a.K; p.nflows = a.nflows; p.B = a.B;
    p.M = a.nflows == 2 ? 2 * a.B : a.B;
    p.row_step = a.nflows == 2 ? 1 : 2;
    p.epi = a.epi; p.out_f32 = a.out_f32; p.h = a.h; p.x_out = a.x_out; p.cpl = a.cpl; p.q_out = a.q_out;
    p.kc = a.kc; p.vc = a.vc; p.len = a.len; p.H = a.H; p.Dh = a.Dh; p.S_max = a.S_max; p.status = a.status;
    p.part = a.part; p.ln_gain = a.ln_gain; p.eps = a.eps;
    p.kw = a.K;
    if (a.dtype == DF_F32) {
        if (p.M > 16) return hipErrorInvalidValue;
        if (a.epi == EPI_RESID_LN && (!a.part || a.N > 4096)) return hipErrorInvalidValue;
        (void)hipGetLastError();
        hipLaunchKernelGGL(gemv_f32, dim3((a.N + 3) / 4), dim3(256), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return finish(p, 1, s);
    }
    if (p.M > 128 || (a.K % 256) != 0) return hipErrorInvalidValue;
    const GemvPlan pl = plan_gemv(a.dtype, a.N, a.K, p.M);
    if ((pl.S > 1 || a.epi == EPI_RESID_LN) && !a.part) return hipErrorInvalidValue;
    if (a.epi == EPI_RESID_LN && a.N > 4096) return hipErrorInvalidValue;
    hipError_t e;
    switch (pl.MT) {
        case 1: e = launch_bf16<1>(p, pl, s); break;
        case 2: e = launch_bf16<2>(p, pl, s); break;
        case 4: e = launch_bf16<4>(p, pl, s); break;
        default: e = launch_bf16<8>(p, pl, s); break;
    }
    if (e != hipSuccess) return e;
    return finish(p, pl.S, s);
}

}  // namespace dfk
