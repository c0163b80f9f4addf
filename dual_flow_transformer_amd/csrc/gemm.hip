// Tiled bf16 matrix-core GEMM for the primary prefill (many rows at once):
// Y[r][n] = sum_k X[r][k] W[n][k], X fp32 rows, W bf16 in the 16x32 fragment
// layout (mfma_tile.h). Prefill costs exactly a standard Transformer over the
// prompt (gist.science/es/paper/2608.12385, "Costes de Inferencia vs.
// Entrenamiento"), so this path is bound by the matrix cores, not by HBM.
//
// Workgroup tile: 128 weight rows x 128 activation rows, 4 waves in a 2x2
// grid of 64 x 64 each (4 x 4 v_mfma_f32_16x16x32_bf16 tiles). Per 64-wide
// k step the activation tile is split into bf16 hi/lo parts into LDS
// (double buffered, the next step's fp32 values already in registers) and
// every wave takes its weight fragments straight from HBM/L2 (each
// fragment is one contiguous 1 KiB piece), the next step's in flight. Both
// activation parts go through the matrix cores into one fp32 accumulator,
// as in the decode projections. Epilogues: store, GELU, residual add.
#include "df_device.h"
#include "df_internal.h"
#include "mfma_tile.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

using tile::bf16x8;
using tile::f32x4;
using tile::u32x4;

constexpr int GT = 128;          // tile edge (weight rows and activation rows)
constexpr int GK = 64;           // k per step
constexpr int GXS = GK + 8;      // LDS row pitch (bf16 elements)
constexpr int GTHREADS = 256;
constexpr int XF4 = GT * GK / 4 / GTHREADS;   // fp32 float4 per thread per step (8)

struct GemmParams {
    const float* x;     // [R][K]
    const bf16_t* w;    // [N][K] fragment layout
    int R, N, K;
    int epi;            // GEMM_STORE / GEMM_GELU / GEMM_RESID
    float* y;           // [R][N] (STORE, GELU) or the residual rows h (RESID)
};

__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

constexpr size_t kGemmLds = (size_t)2 * 2 * GT * GXS * sizeof(bf16_t);

__global__ __launch_bounds__(GTHREADS) void gemm_bf16(GemmParams p) {
    extern __shared__ bf16_t lds[];   // [buffer][hi/lo][row][k]
    auto xs = [&](int buf, int part) { return lds + (size_t)(buf * 2 + part) * GT * GXS; };
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int wn = wv & 1, wm = wv >> 1;
    const int n0 = blockIdx.x * GT, r0 = blockIdx.y * GT;
    const int KB = p.K / 32, NT16 = p.N / 16, nsteps = p.K / GK;

    // activation tile loads: thread i covers rows (i / 16) + 16 j, columns 4 (i % 16)
    auto load_x = [&](int step, float4 (&v)[XF4]) {
        #pragma unroll
        for (int j = 0; j < XF4; ++j) {
            const int e = tid + j * GTHREADS;
            const int row = e >> 4, c4 = e & 15;
            const int r = min(r0 + row, p.R - 1);
            v[j] = *reinterpret_cast<const float4*>(p.x + (size_t)r * p.K + step * GK + 4 * c4);
        }
    };
    auto store_x = [&](int buf, const float4 (&v)[XF4]) {
        #pragma unroll
        for (int j = 0; j < XF4; ++j) {
            const int e = tid + j * GTHREADS;
            const int row = e >> 4, c4 = e & 15;
            uint2 hv, lv;
            df::split_hi_lo(v[j], hv, lv);
            *reinterpret_cast<uint2*>(xs(buf, 0) + row * GXS + 4 * c4) = hv;
            *reinterpret_cast<uint2*>(xs(buf, 1) + row * GXS + 4 * c4) = lv;
        }
    };
    // weight fragments of this wave: 4 tiles of 16 rows x 2 k-blocks of 32
    auto load_w = [&](int step, u32x4 (&a)[4][2]) {
        #pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int t16 = min((n0 + wn * 64 + nt * 16) / 16, NT16 - 1);
            const bf16_t* q = p.w + (((size_t)t16 * KB + step * 2) * 64 + lane) * 8;
            #pragma unroll
            for (int kb = 0; kb < 2; ++kb) a[nt][kb] = *reinterpret_cast<const u32x4*>(q + kb * 512);
        }
    };

    f32x4 acc[4][4];
    #pragma unroll
    for (int i = 0; i < 4; ++i)
        #pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    float4 xv[XF4];
    u32x4 wa[4][2], wb[4][2];
    load_x(0, xv);
    load_w(0, wa);
    store_x(0, xv);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        const bool more = step + 1 < nsteps;
        if (more) {
            load_x(step + 1, xv);
            load_w(step + 1, wb);
        }
        #pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x8 bh[4], bl[4];
            #pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int o = (wm * 64 + mt * 16 + li) * GXS + kb * 32 + lg * 8;
                bh[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs(buf, 0) + o));
                bl[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs(buf, 1) + o));
            }
            #pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, wa[nt][kb]);
                #pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh[mt], acc[nt][mt], 0, 0, 0);
                    acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl[mt], acc[nt][mt], 0, 0, 0);
                }
            }
        }
        if (more) {
            store_x(buf ^ 1, xv);
            #pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                #pragma unroll
                for (int kb = 0; kb < 2; ++kb) wa[nt][kb] = wb[nt][kb];
        }
        __syncthreads();
    }

    // lane holds D[n = 4 lg + i][r = li] of each 16 x 16 tile
    #pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int n = n0 + wn * 64 + nt * 16 + 4 * lg;
        #pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = r0 + wm * 64 + mt * 16 + li;
            if (r >= p.R || n >= p.N) continue;
            float4 v = make_float4(acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]);
            float4* dst = reinterpret_cast<float4*>(p.y + (size_t)r * p.N + n);
            if (p.epi == GEMM_GELU) {
                v.x = gelu(v.x); v.y = gelu(v.y); v.z = gelu(v.z); v.w = gelu(v.w);
            } else if (p.epi == GEMM_RESID) {
                const float4 h = *dst;
                v.x += h.x; v.y += h.y; v.z += h.z; v.w += h.w;
            }
            *dst = v;
        }
    }
}

}  // namespace

hipError_t gemm(const float* x, const void* w, int R, int N, int K, int epi, float* y, hipStream_t s) {
    if (R < 1 || N < 16 || N % 16 || K < GK || K % GK) return hipErrorInvalidValue;
    GemmParams p{x, reinterpret_cast<const bf16_t*>(w), R, N, K, epi, y};
    hipError_t e = tile::allow_lds(reinterpret_cast<const void*>(&gemm_bf16), kGemmLds);
    if (e != hipSuccess) return e;
    (void)hipGetLastError();
    hipLaunchKernelGGL(gemm_bf16, dim3((N + GT - 1) / GT, (R + GT - 1) / GT), dim3(GTHREADS), kGemmLds, s, p);
    return hipGetLastError();
}

}  // namespace dfk
