// Host-side launchers of the dual-flow decode kernels (not exported).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfk {

// Launch kernel fn (its arguments given as pointers in args) on stream s.
// With events, the dispatch itself takes the start and stop timestamps
// (hipExtLaunchKernel), so timing adds no marker packets between kernels.
inline hipError_t launch_timed(const void* fn, dim3 grid, dim3 block, void** args, size_t lds, hipStream_t s,
                               hipEvent_t start, hipEvent_t stop) {
    (void)hipGetLastError();
    if (start || stop) return hipExtLaunchKernel(fn, grid, block, args, lds, s, start, stop, 0);
    return hipLaunchKernel(fn, grid, block, args, lds, s);
}

// ---------------------------------------------------------------------------
// Shared-K/V dual-query attention (split over key chunks, then merged).
// ---------------------------------------------------------------------------
struct AttnArgs {
    int dtype;                // DF_F32 / DF_BF16 (cache storage)
    const void* k;            // cache of one layer: [B][H][S_max][Dh]
    const void* v;
    int B, H, S_max, Dh;
    const float* q;           // [B][2][H][Dh] (flow 1 raw if a != nullptr)
    const float* a;           // [H*Dh] or nullptr: Q2 = Q2raw + a*Q1
    const int32_t* nkeys;     // keys attended by sequence b: nkeys[b] + nkeys_add
    int nkeys_add;
    int nflows;               // 2 = both flows, 1 = primary only
    float* part;              // workspace, attention_part_floats() floats (chunk table and
                              // per-chunk partial results of this call)
    float* o_f32;             // [B][2][H][Dh] fp32 output or nullptr
    float* lse;               // [B][2][H] or nullptr
    float* o_rows;            // [2B][H*Dh] fp32 output rows (projection input), or nullptr
    hipEvent_t ev_start;      // optional events: start and stop timestamps of the partial pass
    hipEvent_t ev_stop;
    // Fused finish of the Q/K/V projection (qkv_part != nullptr; then q is unused and
    // nkeys_add must be 1): q1, q2raw and the primary K/V of the new position
    // nkeys[b] are the slice sums of the projection's EPI_PART partials
    // [qkv_S][M][3*H*Dh] (M = 2B rows with both flows, else B), added in a fixed order
    // (deterministic, the same for both flows); the new K/V row is rounded to the cache type,
    // written at position nkeys[b] (when 0 <= nkeys[b] < S_max; else bit 0 of
    // status[0] is set) and attended from registers.
    const float* qkv_part;
    int qkv_S;
    int32_t* status;
};
size_t attention_part_floats(int B, int H, int S_max, int Dh);
// Partial-result slots of one launch at most, and the largest
// attention_part_floats (head_dim 128).
constexpr int kAttnMaxSlots = 16384;
constexpr size_t kAttnPartFloatsMax = 256 + (size_t)kAttnMaxSlots * (4 + 2 * 128);
// Whether B sequences x H heads fit the slot bound on the current device.
bool attention_fits(int B, int H);
hipError_t attention(const AttnArgs& a, hipStream_t s);
// df_attention_dual after its argument checks; with timed, the launch takes
// the kernel-timing events when timing is enabled (df_timing_enable).
int attention_dual_entry(int dtype, const void* d_k, const void* d_v, int batch, int n_heads, int max_seq,
                         int head_dim, const int32_t* d_len, const float* d_q, const float* d_a, float* d_o,
                         float* d_lse, void* d_ws, size_t ws_bytes, void* stream, bool timed);

// ---------------------------------------------------------------------------
// Row operations
// ---------------------------------------------------------------------------
// Mixture head over logits [B][2][V]; mode: DF_MIX_*. With len_inc, also
// len_inc[b] += 1 for each row once it is done.
hipError_t mix_head(const float* logits, int B, int V, int mode, float* p_mix, float* alpha,
                    int32_t* next_tok, hipStream_t s, int32_t* len_inc = nullptr);
// Mixture head over R row pairs (l1 + i V, l2 + i V) of a prefill-style
// chunk (row i = b * Tc + t); outputs at row (b * T + t0 + t) of [B][T]
// buffers; logits_out [B][T][2][V] may be NULL.
hipError_t mix_rows(const float* l1, const float* l2, int R, int V, int mode, int Tc, int T, int t0,
                    float* logits_out, float* p_mix, float* alpha, int32_t* next_tok, hipStream_t s);

// K/V write at explicit positions (values fp32 [B][H][Dh]).
hipError_t kv_append(int dtype, void* k, void* v, int B, int H, int S_max, int Dh,
                     const int32_t* pos, const float* dk, const float* dv, int32_t* status,
                     hipStream_t s);

// len[b] += inc.
hipError_t len_add(int32_t* len, int B, int inc, hipStream_t s);

// h[2b+f] = E_f[tok[b*tok_stride]] + P[len[b]] (fp32), then x = LN(h; g) (fp32).
// Token ids outside [0, V) are clamped and flagged (status bit 1).
hipError_t embed_ln(int dtype, const void* emb0, const void* emb1, const void* pos_emb,
                    const int32_t* tok, int tok_stride, const int32_t* len, int B, int d, int S_max,
                    int V, int nflows, const float* g, float eps, float* h, void* x, int32_t* status,
                    hipStream_t s);

// Residual rows are summarised per segment of kStatSeg columns as (mean, M2)
// pairs, stats[(r * nseg + seg) * 2 + {0, 1}] for stacked row r, nseg =
// ceil(d / kStatSeg); a LayerNorm then needs no further pass over the row.
constexpr int kStatSeg = 256;
constexpr int kMaxSeg = 16;   // d <= 4096
__host__ __device__ inline int stat_segs(int d) { return (d + kStatSeg - 1) / kStatSeg; }

// x[r] = LN(h[r]; g) (fp32) from the per-segment statistics of h.
hipError_t ln_apply(const float* h, const float* stats, const float* g, float eps, int B, int d, int nflows,
                    float* x, hipStream_t s);

// ---------------------------------------------------------------------------
// Stacked-row GEMV: Y[m][n] = sum_k X[m][k] W[n][k], m over the stacked rows
// in use, with a fused epilogue.
// ---------------------------------------------------------------------------
enum EpiKind {
    EPI_STORE = 0,     // out_f32[m][n] = y
    EPI_QKV = 1,       // Q rows (+ a coupling) to q_out, primary K/V appended to the cache
    EPI_GELU_B = 2,    // g = GELU(y), g2 += b*g1, g to x_out
    EPI_RESID = 3,     // (optional c coupling) h[m][n] += y; per-segment statistics of h to stats_out
    EPI_PART = 4,      // bf16 only: the k-slice partial sums to part[s][m][n] (every S), no finish;
                       // the consumer sums the slices in slice order (attention with AttnArgs::qkv_part)
};

struct GemvArgs {
    int dtype;
    const void* x;        // [2B][K] stacked rows, fp32 (with x_stats: residual rows to normalise)
    const float* x_stats; // bf16 only: per-segment statistics of x; the rows enter as LN(x; x_gain)
    const float* x_gain;
    const void* w;        // bf16: [N][K] in the 16x32 fragment layout; fp32: row-major [N][K]
    int N, K;
    int B;                // sequences
    int nflows;           // 2 or 1 (1: only rows 2b are read and written)
    int epi;
    // epilogue operands
    float* out_f32;       // EPI_STORE: [2B][N]
    float* h;             // EPI_RESID: [2B][N] residual
    float* stats_out;     // EPI_RESID: per-segment statistics of the updated rows
    float* x_out;         // EPI_GELU_B: [2B][N] fp32
    const float* cpl;     // a (QKV), b (GELU_B), c (RESID_LN) or nullptr
    float* q_out;         // EPI_QKV: [2B][d] fp32
    void* kc;             // EPI_QKV: cache of this layer [B][H][S_max][Dh]
    void* vc;
    const int32_t* len;   // EPI_QKV: write position per sequence
    int H, Dh, S_max;
    int32_t* status;      // EPI_QKV: flag when a position is out of range
    float* part;          // split-K partial sums (plan_gemv(...).part_floats floats)
    float eps;            // LayerNorm epsilon (x_stats)
    int slice_rows;       // bf16: stacked rows the k-slicing is planned for (0: the rows in use);
                          // calls with the same slice_rows sum every output over the same slices
};
struct GemvPlan {
    int MT;               // 16-row activation tiles (0: shape not supported)
    int variant;          // kernel shape
    int ks, S;            // k-slice width and count
    int grid;             // workgroups
    int halves;           // 2: rows 0-63 and 64-127 in two workgroups per (row tiles, k-slice)
    size_t lds, part_floats;   // dynamic LDS bytes; partial-sum floats
};
// M: stacked rows in use; M_slices (>= M, else taken as M): the row count whose
// plan fixes the k-slice width.
GemvPlan plan_gemv(int dtype, int N, int K, int M, int M_slices = 0);
hipError_t gemv(const GemvArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Tiled GEMM for prefill: y[r][n] = sum_k x[r][k] w[n][k]; w bf16 [N][K] and
// x as bf16 hi / lo planes [ceil(R/16)*16][K], all in the fragment layout
// (mfma_tile.h). N % 16 == 0, K % 32 == 0.
// ---------------------------------------------------------------------------
enum GemmEpi {
    GEMM_STORE = 0,        // y = x w^T (fp32 [R][N])
    GEMM_GELU_SPLIT = 1,   // GELU(x w^T) as hi / lo fragment planes yh, yl [R16][N] (N % 32 == 0)
    GEMM_RESID = 2,        // y += x w^T (y: fp32 residual rows [R][N])
    GEMM_QKV = 3,          // N = 3 d: Q columns to y [R][d] (fp32), K / V columns into the bf16 cache
    GEMM_GELU_SPLIT_CPL = 4,   // GELU(x w^T) + vec * (primary planes ph + pl at the same row), as planes
    GEMM_RESID_KEEP = 5,   // keep[r] = x w^T and y += x w^T
    GEMM_RESID_CPL = 6,    // y += x w^T + vec * keep[r]
};
// Coupling operands of the dual forward's aux-row epilogues (row r of the
// aux GEMM pairs with row r of the primary one).
struct GemmCouple {
    const float* vec;     // b_l [N] or c_l [N]
    const uint16_t* ph;   // primary GELU output planes [R16][N] (bf16 hi / lo)
    const uint16_t* pl;
    float* keep;          // primary MLP output [R][N] fp32
};
// Where GEMM_QKV puts K and V: row r = b * Tc + t goes to position
// len[b] + t0 + t of sequence b; positions outside [0, S_max) are skipped
// and flagged (status bit 0).
struct QkvStore {
    uint16_t* kc;         // bf16 [B][H][S_max][Dh], one layer
    uint16_t* vc;
    const int32_t* len;
    int Tc, t0, H, Dh, S_max;
    int32_t* status;
};
// With ev_start / ev_stop the launch takes its own start and stop timestamps.
hipError_t gemm(const void* xh, const void* xl, const void* w, int R, int N, int K, int epi, float* y, void* yh,
                void* yl, hipStream_t s, const QkvStore* kv = nullptr, const GemmCouple* cp = nullptr,
                hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// fp32 rows [R][K] -> hi / lo fragment planes (K % 32 == 0).
hipError_t split_rows(const float* x, int R, int K, void* xh, void* xl, hipStream_t s);

// ---------------------------------------------------------------------------
// Prefill row kernels (rows r = b * Tc + t of one chunk of Tc positions
// t0 .. t0 + Tc - 1 per sequence, sequence b at position len[b] + t0 + t).
// ---------------------------------------------------------------------------
// h[r] = primary token embedding + position row (fp32); with emb_aux also
// the aux rows h[R16 + r] from the aux embedding.
hipError_t prefill_embed_rows(const void* emb, const void* pos_emb, const int32_t* tok, int T, int t0, int Tc,
                              const int32_t* len, int B, int d, int S_max, int V, float* h, int32_t* status,
                              hipStream_t s, const void* emb_aux = nullptr, int R16 = 0);
// LayerNorm(h[r]) * g as hi / lo fragment planes xh, xl [R16][d]; d <= 4096, d % 32 == 0.
hipError_t prefill_layer_norm(const float* h, const float* g, float eps, int R, int d, void* xh, void* xl,
                              hipStream_t s);
// Causal attention of the chunk queries q [R][H * Dh] (fp32) over the bf16
// cache: row r, head h = softmax over keys 0 .. len[b] + t0 + t, written as
// hi / lo fragment planes oh, ol [R16][H * Dh]. Dh == 128.
// With q2 (aux raw queries [R][H * Dh]) both flows: the aux query is
// q2 + a * q (a may be NULL) and its output rows sit at R16 + r.
hipError_t prefill_attention(const float* q, int B, int Tc, int t0, const int32_t* len, int H, int Dh, int S_max,
                             const void* kc, const void* vc, void* oh, void* ol, hipStream_t s,
                             const float* q2 = nullptr, const float* a = nullptr, int R16 = 0,
                             hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// ---------------------------------------------------------------------------
// MoE with router replay
// ---------------------------------------------------------------------------
struct MoeArgs {
    int dtype;
    float* h;               // [2B][d] residual rows: normalised for the router, then updated
    const float* stats;     // per-segment statistics of h
    const float* g_ln;      // gain of the norm before the MoE MLP
    const void* w_router;   // [E][d] (fragment layout)
    const float* r1_given;  // [B][E] primary logits supplied, or nullptr
    const void* w_up;       // [E][Fe][d]  (fragment layout per expert)
    const void* w_down;     // [E][d][Fe]  (fragment layout per expert)
    const float* cpl_b;     // [Fe]
    const float* cpl_c;     // [d]
    int B, d, E, k, Fe, nflows;
    int ka;                 // aux fan-out: first ka experts of the primary ranking
    float eps;
    const float* g_next;    // gain of the next norm
    float* x_next;          // [2B][d] LN(h; g_next)
    int32_t* ids_out;       // [B][max(k, ka)] or nullptr
    // workspace (kr = max(k, ka) ranks per sequence, kk of them in use)
    float* x;               // [2B][d] LN(h; g_ln) rows (the experts' input)
    int32_t* ids;           // [B][kr]
    float* gates;           // [B][2][kr], zero beyond a flow's fan-out
    float* g_rows;          // [B*kk][2][Fe] fp32, row 2 (b kk + j) + f
    float* y_rows;          // [B*kk][2][d]
};
hipError_t moe(const MoeArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Row-major bf16 [n_mats][rows][cols] to the 16x32 fragment layout.
// ---------------------------------------------------------------------------
hipError_t pack_weights(const void* src, void* dst, long n_mats, int rows, int cols, hipStream_t s);

}  // namespace dfk
