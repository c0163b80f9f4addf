// Tiled bf16 matrix-core GEMM for the primary prefill (many rows at once):
// Y[r][n] = sum_k X[r][k] W[n][k]. Prefill costs exactly a standard
// Transformer over the prompt (gist.science/es/paper/2608.12385, "Costes de
// Inferencia vs. Entrenamiento"), so this path is bound by the matrix cores,
// not by HBM.
//
// Both operands arrive in the 16 x 32 fragment layout (mfma_tile.h): W as
// bf16 [N][K], X as two bf16 planes [R][K], hi = rne(x) and lo = rne(x - hi)
// of the fp32 activation, written that way by the kernel that produces X
// (LayerNorm, attention, the GELU epilogue, or split_rows below). Every
// operand fetch, global or LDS, is then one contiguous 1 KiB piece per wave.
//
// Workgroup tile: 256 weight rows x 256 activation rows, 8 waves in a 2 x 4
// grid of 128 x 64 each (8 x 4 v_mfma_f32_16x16x32_bf16 tiles, both
// activation parts into one fp32 accumulator). Per 32-wide k block the
// workgroup stages 48 fragments (16 of W, 16 + 16 of X) in LDS with
// direct global-to-LDS loads (each wave-wide load lands as one 1 KiB piece),
// three stages deep: blocks kb + 1 and kb + 2 are in flight while the matrix
// cores work on block kb. Epilogues: fp32 store, residual add, GELU written
// back as hi/lo fragment planes for the next GEMM, or the Q/K/V split (Q
// rows fp32, K and V rounded to bf16 straight into the cache); for the aux
// rows of the dual forward, the b coupling after the GELU and the c
// coupling on the MLP output, each reading the primary row's value.
#include "df_device.h"
#include "df_internal.h"
#include "mfma_tile.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

using tile::bf16x8;
using tile::f32x4;
using tile::u32x4;
using tile::frag_off;

constexpr int TT = 256;                   // tile edge (weight rows and activation rows)
constexpr int TT16 = TT / 16;             // 16-row fragments per tile edge
constexpr int NWAVE = 8;
constexpr int NTHREADS = 64 * NWAVE;
constexpr int PIECES = 3 * TT16;          // fragments staged per k block (W, X hi, X lo)
constexpr int PPW = PIECES / NWAVE;       // fragments per wave (6)
constexpr int FRAG = 512;                 // bf16 elements per fragment (1 KiB)
constexpr int NSTAGE = 3;
constexpr size_t kGemmLds = (size_t)NSTAGE * PIECES * FRAG * sizeof(bf16_t);   // 144 KiB

// s_waitcnt with vmcnt <= n (n < 16), expcnt and lgkmcnt unconstrained.
#define GEMM_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

struct GemmParams {
    const bf16_t* xh;   // [R16][K] fragment layout, R16 = ceil(R / 16) * 16
    const bf16_t* xl;
    const bf16_t* w;    // [N][K] fragment layout
    int R, N, K;
    int epi;            // GEMM_STORE / GEMM_RESID: y fp32 [R][N]; GEMM_GELU_SPLIT: yh / yl planes [R16][N];
                        // GEMM_QKV: y fp32 Q rows [R][N/3], K/V to the cache
    float* y;
    bf16_t* yh;
    bf16_t* yl;
    QkvStore kv;
    GemmCouple cp;
};

__device__ __forceinline__ float gelu(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_bf16(GemmParams p) {
    extern __shared__ u32x4 lds[];   // [stage][piece][lane]
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wn = wv & 1, wr = wv >> 1;           // 128 weight rows x 64 activation rows per wave
    const int KB = p.K >> 5, NT16 = p.N >> 4, RT16 = (p.R + 15) >> 4;
    // XCD-aware order: consecutive workgroups go to different XCDs, so give
    // each XCD a contiguous band of tiles (shared activation rows in its L2).
    const int gx = gridDim.x, total = gx * gridDim.y;
    int id = blockIdx.x + gx * blockIdx.y;
    if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
    const int n0 = (id % gx) * TT16, r0 = (id / gx) * TT16;   // first 16-row fragment of each edge

    // this wave's share of the staged fragments: piece q = wv * PPW + j
    const bf16_t* src[PPW];
    #pragma unroll
    for (int j = 0; j < PPW; ++j) {
        const int q = wv * PPW + j;
        const bf16_t* base;
        int t16;
        if (q < TT16) { base = p.w; t16 = min(n0 + q, NT16 - 1); }
        else if (q < 2 * TT16) { base = p.xh; t16 = min(r0 + q - TT16, RT16 - 1); }
        else { base = p.xl; t16 = min(r0 + q - 2 * TT16, RT16 - 1); }
        src[j] = base + ((size_t)t16 * KB * 64 + lane) * 8;
    }
    // block kb of this wave's pieces -> stage st (global_load_lds: lane i of
    // the wave lands at byte 16 i of the piece)
    auto issue = [&](int kb, int st) {
        #pragma unroll
        for (int j = 0; j < PPW; ++j)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(src[j] + (size_t)kb * FRAG),
                (__attribute__((address_space(3))) void*)(lds + ((size_t)st * PIECES + wv * PPW + j) * 64), 16, 0,
                0);
    };

    f32x4 acc[8][4];
    #pragma unroll
    for (int i = 0; i < 8; ++i)
        #pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    issue(min(1, KB - 1), 1);
    int st = 0;
    for (int kb = 0; kb < KB; ++kb) {
        GEMM_WAIT_VM(PPW);       // this wave's pieces of block kb have landed (kb + 1 may be in flight)
        // ... and every other wave's; all are done with block kb - 1. A bare
        // barrier: the waits above are exact, where a fenced one would drain
        // the loads still in flight for block kb + 1.
        asm volatile("s_barrier" ::: "memory");
        issue(min(kb + 2, KB - 1), st == 0 ? 2 : st - 1);   // stage of block kb - 1 (clamped: always PPW loads)
        const u32x4* S = lds + (size_t)st * PIECES * 64;
        // every operand fragment of the block is read up front, in the order the
        // matrix cores consume them (hi parts first), so each product waits only
        // for its own operands and the lo parts land behind the 32 hi products
        bf16x8 a[8], bh[4], bl[4];
        bh[0] = __builtin_bit_cast(bf16x8, S[(TT16 + wr * 4) * 64 + lane]);
        #pragma unroll
        for (int nt = 0; nt < 8; ++nt) a[nt] = __builtin_bit_cast(bf16x8, S[(wn * 8 + nt) * 64 + lane]);
        #pragma unroll
        for (int mt = 1; mt < 4; ++mt) bh[mt] = __builtin_bit_cast(bf16x8, S[(TT16 + wr * 4 + mt) * 64 + lane]);
        #pragma unroll
        for (int mt = 0; mt < 4; ++mt) bl[mt] = __builtin_bit_cast(bf16x8, S[(2 * TT16 + wr * 4 + mt) * 64 + lane]);
        #pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            #pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[nt], bh[mt], acc[nt][mt], 0, 0, 0);
        #pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            #pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[nt], bl[mt], acc[nt][mt], 0, 0, 0);
        // schedule: ten LDS reads (bh[0], a[], bh[1]), the first eight products,
        // the six other reads, the other 56 products; fewer than 16 reads are
        // ever outstanding, so each product waits only for its own operands
        // (the compiler's own order reuses operand registers and waits for
        // every read three times per block)
        __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 56, 0);
        st = st == 2 ? 0 : st + 1;
    }
    GEMM_WAIT_VM(0);             // no load still landing when the wave leaves

    // lane holds D[n = 4 lg + i][r = li] of each 16 x 16 tile
    const int li = lane & 15, lg = lane >> 4;
    #pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const int n = (n0 + wn * 8 + nt) * 16 + 4 * lg;
        #pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = (r0 + wr * 4 + mt) * 16 + li;
            if (r >= p.R || n >= p.N) continue;
            float4 v = make_float4(acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]);
            if (p.epi == GEMM_QKV) {
                const int d = p.N / 3;
                if (n < d) {
                    *reinterpret_cast<float4*>(p.y + (size_t)r * d + n) = v;
                    continue;
                }
                // K / V columns: rounded to bf16 into the cache of sequence
                // b = r / Tc at position len[b] + t0 + r % Tc
                const QkvStore& q = p.kv;
                const int b = r / q.Tc, pos = q.len[b] + q.t0 + (r - b * q.Tc);
                if (pos < 0 || pos >= q.S_max) {
                    if (q.status) q.status[0] |= 1;
                    continue;
                }
                const int j = n - d - (n >= 2 * d ? d : 0), hh = j / q.Dh, e = j - hh * q.Dh;
                bf16_t* cache = n >= 2 * d ? q.vc : q.kc;
                *reinterpret_cast<uint2*>(cache + (((size_t)b * q.H + hh) * q.S_max + pos) * q.Dh + e) =
                    make_uint2(df::pack_bf16x2(v.x, v.y), df::pack_bf16x2(v.z, v.w));
            } else if (p.epi == GEMM_GELU_SPLIT || p.epi == GEMM_GELU_SPLIT_CPL) {
                v.x = gelu(v.x); v.y = gelu(v.y); v.z = gelu(v.z); v.w = gelu(v.w);
                const size_t o = frag_off(r, n, p.N);
                if (p.epi == GEMM_GELU_SPLIT_CPL) {   // + b * the primary row's GELU output
                    const uint2 qh = *reinterpret_cast<const uint2*>(p.cp.ph + o);
                    const uint2 ql = *reinterpret_cast<const uint2*>(p.cp.pl + o);
                    const float4 b = *reinterpret_cast<const float4*>(p.cp.vec + n);
                    v.x = fmaf(b.x, df::bf16_lo(qh.x) + df::bf16_lo(ql.x), v.x);
                    v.y = fmaf(b.y, df::bf16_hi(qh.x) + df::bf16_hi(ql.x), v.y);
                    v.z = fmaf(b.z, df::bf16_lo(qh.y) + df::bf16_lo(ql.y), v.z);
                    v.w = fmaf(b.w, df::bf16_hi(qh.y) + df::bf16_hi(ql.y), v.w);
                }
                uint2 hv, lv;
                df::split_hi_lo(v, hv, lv);
                *reinterpret_cast<uint2*>(p.yh + o) = hv;
                *reinterpret_cast<uint2*>(p.yl + o) = lv;
            } else {
                float4* dst = reinterpret_cast<float4*>(p.y + (size_t)r * p.N + n);
                if (p.epi == GEMM_RESID_KEEP)        // the primary MLP output, kept for the c coupling
                    *reinterpret_cast<float4*>(p.cp.keep + (size_t)r * p.N + n) = v;
                if (p.epi == GEMM_RESID_CPL) {       // + c * the primary row's MLP output
                    const float4 y1 = *reinterpret_cast<const float4*>(p.cp.keep + (size_t)r * p.N + n);
                    const float4 c = *reinterpret_cast<const float4*>(p.cp.vec + n);
                    v.x = fmaf(c.x, y1.x, v.x); v.y = fmaf(c.y, y1.y, v.y);
                    v.z = fmaf(c.z, y1.z, v.z); v.w = fmaf(c.w, y1.w, v.w);
                }
                if (p.epi != GEMM_STORE) {
                    const float4 h = *dst;
                    v.x += h.x; v.y += h.y; v.z += h.z; v.w += h.w;
                }
                *dst = v;
            }
        }
    }
}

// fp32 rows [R][K] (row-major) -> hi / lo fragment planes; one thread per
// eight consecutive k of one row.
__global__ __launch_bounds__(256) void split_rows_kernel(const float* x, int R, int K, bf16_t* xh, bf16_t* xl) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per_row = K >> 3;
    if (i >= (size_t)R * per_row) return;
    const int r = (int)(i / per_row), k = (int)(i - (size_t)r * per_row) * 8;
    const float4 a = *reinterpret_cast<const float4*>(x + (size_t)r * K + k);
    const float4 b = *reinterpret_cast<const float4*>(x + (size_t)r * K + k + 4);
    uint2 h0, l0, h1, l1;
    df::split_hi_lo(a, h0, l0);
    df::split_hi_lo(b, h1, l1);
    const size_t o = frag_off(r, k, K);
    *reinterpret_cast<u32x4*>(xh + o) = (u32x4){h0.x, h0.y, h1.x, h1.y};
    *reinterpret_cast<u32x4*>(xl + o) = (u32x4){l0.x, l0.y, l1.x, l1.y};
}

}  // namespace

hipError_t gemm(const void* xh, const void* xl, const void* w, int R, int N, int K, int epi, float* y, void* yh,
                void* yl, hipStream_t s, const QkvStore* kv, const GemmCouple* cp, hipEvent_t ev_start,
                hipEvent_t ev_stop) {
    if (R < 1 || N < 16 || N % 16 || K < 32 || K % 32 || epi < GEMM_STORE || epi > GEMM_RESID_CPL)
        return hipErrorInvalidValue;
    const bool split = epi == GEMM_GELU_SPLIT || epi == GEMM_GELU_SPLIT_CPL;
    if (split ? (!yh || !yl || N % 32) : !y) return hipErrorInvalidValue;
    if (epi == GEMM_QKV && (!kv || N % 3 || (N / 3) % 16 || kv->Dh % 4 || kv->Tc < 1 || R % kv->Tc))
        return hipErrorInvalidValue;
    if ((epi == GEMM_GELU_SPLIT_CPL && (!cp || !cp->vec || !cp->ph || !cp->pl)) ||
        (epi == GEMM_RESID_KEEP && (!cp || !cp->keep)) || (epi == GEMM_RESID_CPL && (!cp || !cp->vec || !cp->keep)))
        return hipErrorInvalidValue;
    GemmParams p{reinterpret_cast<const bf16_t*>(xh), reinterpret_cast<const bf16_t*>(xl),
                 reinterpret_cast<const bf16_t*>(w), R, N, K, epi, y, reinterpret_cast<bf16_t*>(yh),
                 reinterpret_cast<bf16_t*>(yl), kv ? *kv : QkvStore{}, cp ? *cp : GemmCouple{}};
    hipError_t e = tile::allow_lds(reinterpret_cast<const void*>(&gemm_bf16), kGemmLds);
    if (e != hipSuccess) return e;
    void* args[] = {&p};
    return launch_timed(reinterpret_cast<const void*>(&gemm_bf16), dim3((N + TT - 1) / TT, (R + TT - 1) / TT),
                        dim3(NTHREADS), args, kGemmLds, s, ev_start, ev_stop);
}

hipError_t split_rows(const float* x, int R, int K, void* xh, void* xl, hipStream_t s) {
    if (R < 1 || K < 32 || K % 32) return hipErrorInvalidValue;
    const size_t n = (size_t)R * (K / 8);
    (void)hipGetLastError();
    hipLaunchKernelGGL(split_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, R, K,
                       reinterpret_cast<bf16_t*>(xh), reinterpret_cast<bf16_t*>(xl));
    return hipGetLastError();
}

}  // namespace dfk
