/*
 * dualflow.h - C ABI of the Dual-Flow Transformer grouped decode step on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (arXiv 2608.12385, "Dual-Flow Transformers: Decoupling the
 * Primary Prefill Path from Additional Decode Computation"; summarised on
 * gist.science/es/paper/2608.12385, "Resumen Tecnico: Dual-Flow
 * Transformers"): a primary flow, a standard causal Transformer, owns the
 * single persistent K/V cache; an auxiliary flow with its own token
 * embedding runs only from the last prompt position on, shares every
 * attention, MLP and output matrix, couples one way to the primary through
 * per-layer vectors a_l (query), b_l (MLP intermediate) and c_l (MLP
 * output), attends the primary K/V and never writes it; the two output
 * distributions are mixed as p_mix = alpha p_primary + (1 - alpha) p_aux
 * with alpha from the primary's collision probability, at least 0.5; in MoE
 * models the aux flow replays the primary's expert choice with its own gates
 * (section "Mecanismos Clave"). Decode groups both flows so every weight and
 * K/V region is read once (section "Costes de Inferencia vs.
 * Entrenamiento").
 *
 * Conventions for every entry point:
 *  - Pointers prefixed d_ are device memory owned by the caller; host structs
 *    (df_config, df_weights, df_kv) are read during the call only.
 *  - The library never allocates device memory. Scratch space is the
 *    caller's workspace (d_ws, ws_bytes), sized by the *_workspace_bytes
 *    queries, 256-byte aligned. A decode workspace must be zero-filled
 *    before its first use (its first word is the device status word).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns DF_OK or a negative DF_ERR_* code. Host-side
 *    argument checks run before anything is launched; a failed check
 *    launches nothing. DF_ERR_HIP reports a launch error (the HIP error is
 *    left for the caller to read with hipGetLastError).
 *  - Storage dtype (weights, embeddings, K/V): DF_F32 or DF_BF16. Coupling
 *    vectors and LayerNorm gains are always fp32. Activations are fp32 and
 *    accumulation is fp32; appended K/V entries are rounded to the storage
 *    dtype (nearest-even). With DF_BF16 the projections run on bf16 matrix
 *    cores, each fp32 activation entering as a pair of bf16 parts whose sum
 *    is within 2^-17 of it.
 *  - Stacked rows: row 2b is the primary flow of sequence b, row 2b+1 its
 *    aux flow ([B][2][...] layouts below).
 *  - Results are deterministic: no atomics take part in any reduction.
 */
#ifndef DUALFLOW_H
#define DUALFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    DF_OK = 0,
    DF_ERR_NULL = -1,       /* a required pointer is NULL */
    DF_ERR_SHAPE = -2,      /* a size is out of range or unsupported */
    DF_ERR_DTYPE = -3,      /* unknown storage dtype */
    DF_ERR_ALIGN = -4,      /* a pointer is not 16-byte aligned (workspace: 256) */
    DF_ERR_WORKSPACE = -5,  /* workspace smaller than the query returns */
    DF_ERR_KV_FULL = -6,    /* a write position would be >= max_seq */
    DF_ERR_HIP = -7,        /* a HIP launch failed */
    DF_ERR_ARG = -8         /* another invalid argument */
};

enum { DF_F32 = 0, DF_BF16 = 1 };

/* Model variant switches (df_config.variant, bit flags): the ablations of
 * gist.science/es/paper/2608.12385, section "Resultados" (a minimal Dual
 * construction without the cross-flow coupling and without the probability
 * mixture), and the other reading of the alpha floor. */
enum {
    DF_VARIANT_NO_COUPLING = 1,  /* a_l, b_l, c_l not applied (their vectors are not read) */
    DF_VARIANT_AUX_OUTPUT = 2,   /* no mixture: p_mix = p_aux, alpha = 0 */
    DF_VARIANT_ALPHA_HALF = 4    /* alpha = (1 + sum_v p_primary(v)^2) / 2; excludes AUX_OUTPUT */
};

/* Mixture modes of df_mix_head. */
enum { DF_MIX_PRIMARY = 0, DF_MIX_COLLISION = 1, DF_MIX_AUX = 2, DF_MIX_HALF = 3 };

/* Model and batch sizes. n_experts == 0 selects the dense MLP (width ffn);
 * n_experts > 0 selects the MoE MLP (top_k experts of width expert_ffn).
 * top_k_aux (MoE): 0 = the aux flow replays the primary's top_k experts;
 * 1..16 = the aux flow takes the first top_k_aux experts of the primary's
 * ranking, with its own gates (independent expert fan-outs, section
 * "Contribuciones Clave" item 3); the b_l coupling then applies on the
 * experts the primary also ran (ranks below top_k). Must be 0 for dense
 * models.
 * Supported: head_dim in {32, 64, 128}; d_model == n_heads * head_dim;
 * with DF_BF16, d_model, ffn and expert_ffn multiples of 256 and vocab and
 * n_experts multiples of 16; batch <= 64 (stacked rows 2*batch <= 128). */
typedef struct df_config {
    int32_t n_layers;
    int32_t d_model;
    int32_t n_heads;
    int32_t head_dim;
    int32_t ffn;
    int32_t vocab;
    int32_t n_experts;
    int32_t top_k;
    int32_t expert_ffn;
    int32_t batch;
    int32_t max_seq;     /* cache capacity (positions) = rows of pos_emb */
    int32_t dtype;       /* DF_F32 or DF_BF16 */
    float ln_eps;        /* LayerNorm epsilon */
    int32_t variant;     /* DF_VARIANT_* flags, 0 = the full method */
    int32_t top_k_aux;   /* MoE aux expert fan-out, 0 = replay of top_k */
    int32_t prefill_rows; /* rows (batch x positions) per prefill chunk, 0 = DF_PREFILL_ROWS */
} df_config;

/* Parameters, all device pointers, layer-major stacks. Embeddings and
 * position tables are row-major. Projection matrices are [out][in]
 * (w[n][k] multiplies input k into output n): with DF_F32 row-major, with
 * DF_BF16 in the 16x32 fragment layout of df_pack_weights, each matrix of a
 * stack packed on its own (the layout every wave-wide weight load of the
 * bf16 matrix cores reads as one contiguous 1 KiB piece). */
typedef struct df_weights {
    const void* tok_emb[2];    /* [vocab][d]: primary (0), aux (1) */
    const void* pos_emb;       /* [max_seq][d], shared by both flows */
    const float* ln1;          /* [L][d]  gain of the norm before attention */
    const float* ln2;          /* [L][d]  gain of the norm before the MLP */
    const float* lnf;          /* [d]     final norm gain */
    const void* w_qkv;         /* [L][3d][d]: rows Q (h*Dh+i), then K, then V */
    const void* w_o;           /* [L][d][d] */
    const void* w_up;          /* [L][ffn][d]          (dense) */
    const void* w_down;        /* [L][d][ffn]          (dense) */
    const void* w_router;      /* [L][E][d]            (MoE) */
    const void* w_exp_up;      /* [L][E][expert_ffn][d] (MoE) */
    const void* w_exp_down;    /* [L][E][d][expert_ffn] (MoE) */
    const float* cpl_a;        /* [L][d]   query coupling a_l */
    const float* cpl_b;        /* [L][ffn or expert_ffn]  intermediate coupling b_l */
    const float* cpl_c;        /* [L][d]   output coupling c_l */
    const void* w_out;         /* [vocab][d] LM head */
} df_weights;

/* The single persistent K/V cache, written by the primary flow only.
 * k, v: [L][batch][n_heads][max_seq][head_dim] in the storage dtype.
 * len: [batch] int32, positions filled so far (the next write position). */
typedef struct df_kv {
    void* k;
    void* v;
    int32_t* len;
} df_kv;

/* Bytes of workspace df_decode_step and df_prefill_primary need. */
size_t df_workspace_bytes(const df_config* cfg);

/* One grouped decode step, both flows (gist.science/es/paper/2608.12385,
 * sections "Arquitectura Central" and "Mecanismos Clave").
 *  d_tokens [batch]: token of each sequence at position len[b].
 *  aux_on: 1 = dual step; 0 = primary-only step (p_mix = p_primary,
 *    alpha = 1). The primary numerics (logits, cache, expert ids) are bitwise
 *    those of a dual step at every batch size: both modes split every
 *    projection's k range into the same slices (the plan for the 2 * batch
 *    stacked rows) and add them in the same order, and no other reduction
 *    depends on the row count.
 *  d_router_logits [L][batch][n_experts] or NULL: MoE only, primary router
 *    logits supplied by the caller (replacing the primary router output);
 *    NULL computes them from w_router.
 *  d_logits [batch][2][vocab] or NULL: raw logits of both flows (fp32).
 *  d_p_mix [batch][vocab], d_alpha [batch]: the mixture output.
 *  d_next_tok [batch] or NULL: argmax of p_mix, ties to the lowest id.
 *  d_expert_ids [L][batch][max(top_k, top_k_aux)] or NULL: MoE, the
 *    primary's expert ranking by descending logit, ties to the lower id (the
 *    first top_k are the primary's experts; the aux flow uses the first
 *    top_k_aux, or the first top_k when top_k_aux = 0).
 * Appends the primary K/V at len[b] in every layer, then len[b] += 1 (on
 * the device). A sequence whose len[b] >= max_seq is not written and is
 * flagged in the device status (df_device_status). */
int df_decode_step(const df_config* cfg, const df_weights* w, const df_kv* kv,
                   const int32_t* d_tokens, int32_t aux_on, const float* d_router_logits,
                   float* d_logits, float* d_p_mix, float* d_alpha, int32_t* d_next_tok,
                   int32_t* d_expert_ids, void* d_ws, size_t ws_bytes, void* stream);

/* Bytes of workspace df_prefill_primary needs (>= df_workspace_bytes):
 * dense bf16 models with head_dim 128 add room for one chunk of R prompt
 * rows, about R * (3 d + ffn) * 4 bytes (fp32 residual and query rows, the
 * GEMM operands as bf16 hi/lo planes). 0 when the config is invalid. */
size_t df_prefill_workspace_bytes(const df_config* cfg);

/* Default rows (batch x positions) per chunk of the compute-bound prefill. */
#define DF_PREFILL_ROWS 16384

/* Primary-only prefill of T tokens per sequence (d_tokens [batch][T]) at
 * positions len[b] .. len[b]+T-1: the aux flow is skipped in prefill and
 * the primary flow is a standard causal Transformer over the prompt
 * (sections "Arquitectura Central" and "Costes de Inferencia vs.
 * Entrenamiento"). Writes the K/V of every prompt position (rounded to the
 * storage dtype) and advances len[b] by T; no logits are produced.
 *  Dense bf16 models with head_dim 128: the prompt goes through in chunks
 *    of Tc = max(1, min(max_seq, rows / batch)) positions per sequence, rows
 *    = cfg->prefill_rows or DF_PREFILL_ROWS; per chunk and layer the projections are tiled matrix-core
 *    GEMMs over the batch * Tc rows, and a causal attention pass takes each
 *    chunk query over the cached keys 0 .. its own position.
 *  Other models: the kernels of a primary-only decode step, one position at
 *    a time.
 * ws_bytes must be at least df_prefill_workspace_bytes(cfg). Positions at or
 * past max_seq are not written and are flagged in the device status; token
 * ids outside [0, vocab) are clamped and flagged. */
int df_prefill_primary(const df_config* cfg, const df_weights* w, const df_kv* kv,
                       const int32_t* d_tokens, int32_t T, void* d_ws, size_t ws_bytes,
                       void* stream);

/* Bytes of workspace df_forward_dual needs (>= df_workspace_bytes). Dense
 * bf16 models with head_dim 128 add one chunk of both flows' rows, about
 * 2 R (3 d + ffn + vocab) * 4 bytes for R = batch * Tc; others a few rows
 * of outputs. 0 when the config is invalid. */
size_t df_forward_workspace_bytes(const df_config* cfg);

/* Full-sequence dual forward: both flows at every position of T tokens per
 * sequence (d_tokens [batch][T]) at positions len[b] .. len[b]+T-1, as both
 * flows are evaluated along the whole sequence in training (section "Costes
 * de Inferencia vs. Entrenamiento"). The primary flow is the causal
 * Transformer of the prefill and writes K/V of every position; the aux flow
 * forms Q2 = Q2raw + a * Q1 and attends the primary K/V of positions up to
 * its own, with the b / c couplings of each position (sections "Arquitectura
 * Central", "Mecanismos Clave"). Equals T teacher-forced df_decode_step
 * calls with aux_on = 1 (up to rounding order). Advances len[b] by T.
 *  d_logits [batch][T][2][vocab] or NULL; d_p_mix [batch][T][vocab];
 *  d_alpha [batch][T]; d_next_tok [batch][T] or NULL (argmax of p_mix).
 *  Model variants (cfg->variant) apply as in the decode step; MoE models
 *  route every position with the primary router (replay for the aux row).
 *  Dense bf16 models with head_dim 128: chunks of Tc = max(1, min(max_seq,
 *    rows / 2 / batch)) positions (rows = cfg->prefill_rows or
 *    DF_PREFILL_ROWS) through tiled matrix-core GEMMs over the stacked rows
 *    of both flows and one causal attention pass for both query sets.
 *  Other models: one dual step per position with the decode-step kernels.
 * ws_bytes must be at least df_forward_workspace_bytes(cfg). */
int df_forward_dual(const df_config* cfg, const df_weights* w, const df_kv* kv,
                    const int32_t* d_tokens, int32_t T, float* d_logits, float* d_p_mix,
                    float* d_alpha, int32_t* d_next_tok, void* d_ws, size_t ws_bytes,
                    void* stream);

/* Append primary K/V entries to the one persistent cache
 * (gist.science/es/paper/2608.12385, "Arquitectura Central": only the
 * primary flow writes K/V; the aux flow reads the primary's entries and
 * never writes): for each sequence b and head h of one layer,
 * k[layer][b][h][d_pos[b]][:] = round(d_k[b][h][:]) (same for v).
 *  d_k, d_v: fp32 [batch][n_heads][head_dim], rounded to the storage dtype
 *    (nearest-even for bf16).
 *  d_pos: int32 [batch] device positions; entries outside [0, max_seq) are
 *    skipped and set bit 0 of *d_status (int32 device word, may be NULL).
 * The decode step does not call this: with bf16 storage its attention pass
 * forms, rounds and writes the new entry itself (and attends it from
 * registers), with fp32 storage the Q/K/V projection's epilogue writes it.
 * Asynchronous on `stream`; returns DF_ERR_* for bad arguments before any
 * launch. */
int df_kv_append(const df_config* cfg, const df_kv* kv, int32_t layer, const int32_t* d_pos,
                 const float* d_k, const float* d_v, int32_t* d_status, void* stream);

/* The mixture head alone (section "Mecanismos Clave", mixture objective):
 * d_logits [batch][2][vocab] fp32. p_f = softmax(logits_f) over the whole
 * vocabulary; p_mix = alpha p_primary + (1 - alpha) p_aux with, by mode:
 * DF_MIX_COLLISION: alpha = min(1, max(0.5, sum_v p_primary(v)^2));
 * DF_MIX_HALF: alpha = (1 + sum_v p_primary(v)^2) / 2;
 * DF_MIX_AUX: alpha = 0 (p_mix = p_aux);
 * DF_MIX_PRIMARY: alpha = 1 (p_mix = p_primary, aux logits not read).
 * d_next_tok (argmax of p_mix, ties to the lowest id) may be NULL. */
int df_mix_head(const float* d_logits, int32_t batch, int32_t vocab, int32_t mode,
                float* d_p_mix, float* d_alpha, int32_t* d_next_tok, void* stream);

/* Asymmetric shared-K/V attention alone (section "Mecanismos Clave"): for
 * each sequence b and head h both queries attend cache positions
 * 0 .. d_len[b]-1 of the one cache, which is read once for both.
 *  d_k, d_v: [batch][n_heads][max_seq][head_dim] (one layer), storage dtype.
 *  d_q: [batch][2][n_heads][head_dim] fp32, flow 0 = Q1, flow 1 = Q2raw.
 *  d_a: [n_heads*head_dim] or NULL: if given Q2 = Q2raw + a * Q1.
 *  d_o: [batch][2][n_heads][head_dim] fp32 outputs; d_lse: [batch][2][n_heads]
 *  natural-log sum of exp of the scaled scores. Scores are q.k/sqrt(head_dim).
 *  d_len[b] is clamped to [0, max_seq]; a sequence with no keys
 *  (d_len[b] = 0) gets zero outputs and lse = -inf. batch <= 64 and
 *  batch * n_heads <= 16384 - 4 x (compute units), 15360 on the MI355X
 *  (else DF_ERR_SHAPE).
 *  d_ws: df_attention_workspace_bytes bytes (the call's chunk table and
 *  per-chunk partial results; no initial contents needed). */
int df_attention_dual(int32_t dtype, const void* d_k, const void* d_v, int32_t batch,
                      int32_t n_heads, int32_t max_seq, int32_t head_dim, const int32_t* d_len,
                      const float* d_q, const float* d_a, float* d_o, float* d_lse,
                      void* d_ws, size_t ws_bytes, void* stream);

/* df_attention_dual without a workspace argument and without allocating
 * anything, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, results and errors as df_attention_dual; the chunk table and
 * partial results go to a static device array of the library,
 * DF_ATTENTION_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, kept
 * until the process ends. Its address is looked up once per device (on the
 * first call with that device current). Every call on a GPU shares that
 * GPU's array, so calls that overlap on one GPU (different streams, or
 * several host threads) race: order them on one stream. Sizes whose
 * workspace would exceed the array return DF_ERR_WORKSPACE (no supported
 * size does); more than 16384 - 4 x (compute units) sequence-head pairs
 * return DF_ERR_SHAPE, as in df_attention_dual. Never calls hipMalloc or
 * hipFree; no kernel timing. */
#define DF_ATTENTION_NOALLOC_SCRATCH_BYTES 17040384
int df_attention_dual_noalloc(int32_t dtype, const void* d_k, const void* d_v, int32_t batch,
                              int32_t n_heads, int32_t max_seq, int32_t head_dim, const int32_t* d_len,
                              const float* d_q, const float* d_a, float* d_o, float* d_lse, void* stream);

/* Workspace bytes df_attention_dual needs for these sizes. */
size_t df_attention_workspace_bytes(int32_t batch, int32_t n_heads, int32_t max_seq, int32_t head_dim);

/* The stacked-row projection alone (the building block of every shared
 * weight in the step, gist.science/es/paper/2608.12385, "Arquitectura
 * Central": both flows use the same matrices):
 * y[m][n] = sum_k x[m][k] w[n][k] for m < rows.
 *  d_x: fp32 [rows][K]; d_w: [N][K] in `dtype` (DF_F32 row-major, DF_BF16
 *  in the fragment layout of df_pack_weights); d_y: fp32 [rows][N].
 *  rows <= 128: the decode projection (rows even: primary/aux row pairs;
 *  DF_F32: rows <= 16; DF_BF16: K a multiple of 256, N of 16).
 *  DF_BF16 and rows > 128: the tiled matrix-core GEMM of the prefill (any
 *  row count; K a multiple of 32, N of 16).
 *  With DF_BF16 each x element enters the bf16 matrix cores as two bf16
 *  parts whose sum is within 2^-17 of it.
 *  d_ws: df_stacked_gemv_workspace_bytes bytes (split-K partial sums, or for
 *  the tiled GEMM the rows as bf16 hi / lo planes). */
int df_stacked_gemv(int32_t dtype, const float* d_x, const void* d_w, int32_t rows, int32_t N, int32_t K,
                    float* d_y, void* d_ws, size_t ws_bytes, void* stream);

/* Workspace bytes of df_stacked_gemv for these sizes (0 if unsupported). */
size_t df_stacked_gemv_workspace_bytes(int32_t dtype, int32_t rows, int32_t N, int32_t K);

/* Repacks n_mats row-major bf16 matrices [rows][cols] (consecutive in
 * d_src) into the 16x32 fragment layout at d_dst (same size, no overlap):
 * element (n, k) of a matrix goes to
 *   ((n/16 * cols/32 + k/32) * 64 + ((k%32)/8) * 16 + n%16) * 8 + k%8,
 * i.e. each 16-row x 32-column block becomes 64 groups of 8 consecutive k
 * in the order the bf16 matrix-core A operand takes them (group
 * (k%32)/8 * 16 + n%16 belongs to lane of that number). DF_BF16 only;
 * rows % 16 == 0, cols % 32 == 0. Asynchronous on `stream`. */
int df_pack_weights(int32_t dtype, const void* d_src, void* d_dst, int64_t n_mats, int32_t rows, int32_t cols,
                    void* stream);

/* Reads and clears the device status word kept in a decode workspace
 * (bit 0: a K/V write was skipped because len >= max_seq; bit 1: a token
 * id outside [0, vocab) was clamped). Synchronises
 * `stream`. */
int df_device_status(void* d_ws, void* stream, int32_t* status_out);

/* Text of a DF_* return code. */
const char* df_status_str(int code);

/* A measurement instrument, not a step of the method: a plain streaming
 * read of `bytes` bytes at d_src in the launch shape of the decode
 * attention pass (one 4-wave workgroup per compute unit, each wave reading
 * one contiguous share with 16-byte non-temporal loads). Its duration is the
 * read rate that pass, which reads each K/V byte once, can at best reach on
 * the device; small sizes give the fixed cost of one launch.
 *  d_src: device memory, 16-byte aligned; bytes: a multiple of 16 (0 is
 *  allowed). d_out: device uint32 [DF_STREAM_READ_OUT_WORDS]; wave w writes
 *  the XOR of the 32-bit words it read to d_out[w] (w < 4 x compute units),
 *  the other words are untouched: with d_out cleared first, the XOR of all
 *  its words is the XOR of every word of the source.
 * Asynchronous on `stream`. DF_ERR_NULL, DF_ERR_ALIGN (pointer or size),
 * DF_ERR_SHAPE (device with more than DF_STREAM_READ_OUT_WORDS / 4 compute
 * units), DF_ERR_HIP (launch failure). */
#define DF_STREAM_READ_OUT_WORDS 4096
int df_stream_read(const void* d_src, size_t bytes, uint32_t* d_out, void* stream);

/* Kernel timing with HIP events on the launching stream. While enabled,
 * launches of the kernels of class `kclass` (0 = attention partial pass
 * of a decode step, 1 = tiled GEMM of the prefill projections, 2 = causal
 * prefill attention) are counted from 0, and every launch whose count is
 * a multiple of `stride` (>= 1) takes a pair of events as its own start
 * and stop timestamps (hipExtLaunchKernel: no marker packets between
 * kernels). Each timed launch costs a few microseconds more than an
 * untimed one, so a stride above 1 keeps the timed work close to the
 * untimed; a stride that shares no factor with the number of launches
 * per step samples every layer in turn. df_timing_read synchronises the
 * events and returns the summed duration (ms) and the number of timed
 * launches, then disables timing. At most 65536 launches are timed.
 * DF_ERR_ARG for an unknown class or a stride below 1. */
int df_timing_enable(int32_t kclass, int32_t stride);
int df_timing_read(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* DUALFLOW_H */
