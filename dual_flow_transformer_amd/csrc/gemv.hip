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
using tile::RT;
using tile::ROWS;

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
    void* x_out;
    const float* cpl;
    float* q_out;
    void* kc;
    void* vc;
    const int32_t* len;
    int H, Dh, S_max;
    int32_t* status;
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
        case EPI_RESID:
            if (dual && p.cpl) y2 = fmaf(p.cpl[n], y1, y2);   // MLP-output coupling (c_l)
            p.h[r1] += y1;
            if (dual) p.h[r2] += y2;
            break;
        case EPI_GELU_B: {
            const float g1 = gelu(y1);
            T* xo = reinterpret_cast<T*>(p.x_out);
            df::St<T>::st(xo, r1, g1);
            if (dual) {
                float g2 = gelu(y2);
                if (p.cpl) g2 = fmaf(p.cpl[n], g1, g2);          // MLP-intermediate coupling (b_l)
                df::St<T>::st(xo, r2, g2);
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

template <int MT, int KU>
__global__ __launch_bounds__(1024) void gemv_bf16(GParams p) {
    extern __shared__ float red[];   // [NW][RT][MT][4][64]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, NW = blockDim.x >> 6;
    const int n0 = blockIdx.x * ROWS;
    const int li = lane & 15, lg = lane >> 4;
    const bf16_t* W = reinterpret_cast<const bf16_t*>(p.w);
    const bf16_t* X = reinterpret_cast<const bf16_t*>(p.x);
    const bf16_t* wrow[RT];
    #pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n = min(n0 + rt * 16 + li, p.N - 1);
        wrow[rt] = W + (size_t)n * p.K + lg * 8;
    }
    const bf16_t* xrow[MT];
    #pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = min(mt * 16 + li, p.M - 1);
        xrow[mt] = X + (size_t)(m * p.row_step) * p.K + lg * 8;
    }
    f32x4 acc[RT][MT];
    tile::zero<MT>(acc);
    tile::stream_k<MT, KU>(wrow, xrow, MT, wv * p.kw, (wv + 1) * p.kw, acc);
    tile::to_lds<MT>(red, wv, lane, acc);
    __syncthreads();
    const bool dual = p.nflows == 2;
    for (int t = threadIdx.x; t < ROWS * p.B; t += blockDim.x) {
        const int nl = t % ROWS, b = t / ROWS;
        const int n = n0 + nl;
        if (n >= p.N) continue;
        const float y1 = tile::lds_sum<MT>(red, NW, nl, dual ? 2 * b : b);
        const float y2 = dual ? tile::lds_sum<MT>(red, NW, nl, 2 * b + 1) : 0.f;
        epilogue<bf16_t>(p, n, b, y1, y2);
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
hipError_t launch_bf16(GParams& p, hipStream_t s) {
    constexpr int KU = MT <= 2 ? 4 : 2;
    const int nwg = (p.N + ROWS - 1) / ROWS;
    const int nw = tile::pick_waves(nwg, p.K, MT, KU, 4096);
    p.kw = p.K / nw;
    const size_t lds = (size_t)nw * RT * MT * 256 * sizeof(float);
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_bf16<MT, KU>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr_set = true;
    }
    hipLaunchKernelGGL((gemv_bf16<MT, KU>), dim3(nwg), dim3(64 * nw), lds, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t gemv(const GemvArgs& a, hipStream_t s) {
    GParams p;
    p.x = a.x; p.w = a.w; p.N = a.N; p.K = a.K; p.nflows = a.nflows; p.B = a.B;
    p.M = a.nflows == 2 ? 2 * a.B : a.B;
    p.row_step = a.nflows == 2 ? 1 : 2;
    p.epi = a.epi; p.out_f32 = a.out_f32; p.h = a.h; p.x_out = a.x_out; p.cpl = a.cpl; p.q_out = a.q_out;
    p.kc = a.kc; p.vc = a.vc; p.len = a.len; p.H = a.H; p.Dh = a.Dh; p.S_max = a.S_max; p.status = a.status;
    p.kw = a.K;
    if (a.dtype == DF_F32) {
        if (p.M > 16) return hipErrorInvalidValue;
        hipLaunchKernelGGL(gemv_f32, dim3((a.N + 3) / 4), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    const int mt = (p.M + 15) / 16;
    if (mt <= 1) return launch_bf16<1>(p, s);
    if (mt <= 2) return launch_bf16<2>(p, s);
    if (mt <= 4) return launch_bf16<4>(p, s);
    if (mt <= 8) return launch_bf16<8>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace dfk
