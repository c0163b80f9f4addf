// C ABI of the dual-flow grouped decode step: argument checks, workspace
// carving and the per-layer kernel sequence on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/dualflow.h"
#include "df_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kStackedRows = 128;   // df_stacked_gemv: above this, the tiled GEMM

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(int dtype) { return dtype == DF_BF16 ? 2 : 4; }

typedef char* bf16p;   // byte pointer into bf16 hi / lo planes

// Workspace regions (byte offsets from the workspace base).
struct WsLayout {
    size_t status, h, xd, xo, xf, q, part, logits, ids, gates, grows, yrows, gpart,
        stats, total;
};

// Largest split-K partial buffer over the model's GEMVs.
void gemv_scratch(const df_config& c, size_t* part_floats) {
    const bool moe = c.n_experts > 0;
    const int d = c.d_model;
    const int shapes[5][2] = {{3 * d, d}, {d, d}, {moe ? 0 : c.ffn, d}, {d, moe ? 0 : c.ffn},
                              {c.vocab, d}};
    *part_floats = 0;
    for (int M : {2 * c.batch, c.batch}) {
        for (auto& sh : shapes) {
            if (sh[0] <= 0 || sh[1] <= 0) continue;
            const dfk::GemvPlan pl = dfk::plan_gemv(c.dtype, sh[0], sh[1], M, 2 * c.batch);
            const size_t need = pl.part_floats > 0 ? pl.part_floats : (size_t)M * sh[0];
            if (need > *part_floats) *part_floats = need;
        }
    }
}

WsLayout layout(const df_config& c) {
    const size_t es = elem_size(c.dtype);
    const size_t M = 2 * (size_t)c.batch;
    const bool moe = c.n_experts > 0;
    const size_t P = (size_t)c.batch * (moe ? std::max(c.top_k, c.top_k_aux) : 0);
    WsLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
    L.status = take(kAlign);
    L.h = take(M * c.d_model * 4);
    L.xd = take(M * c.d_model * 4);
    L.xo = take(M * c.d_model * 4);
    L.xf = take(moe ? 0 : M * (size_t)c.ffn * 4);
    L.q = take(M * c.d_model * 4);
    L.part = take(dfk::attention_part_floats(c.batch, c.n_heads, c.max_seq, c.head_dim) * 4);
    L.logits = take(M * (size_t)c.vocab * 4);
    L.ids = take(P * 4);
    L.gates = take(P * 2 * 4);
    L.grows = take(P * 2 * (size_t)c.expert_ffn * 4);
    L.yrows = take(P * 2 * (size_t)c.d_model * 4);
    size_t gp = 0;
    gemv_scratch(c, &gp);
    L.gpart = take(gp * 4);
    L.stats = take(M * dfk::stat_segs(c.d_model) * 2 * 4);
    L.total = o;
    return L;
}

// Compute-bound prefill (dense bf16, head_dim 128): chunk of Tc positions
// per sequence, rows r = b * Tc + t.
bool fast_prefill(const df_config& c) { return c.dtype == DF_BF16 && c.n_experts == 0 && c.head_dim == 128; }
int prefill_chunk(const df_config& c) {
    const int rows = c.prefill_rows > 0 ? c.prefill_rows : DF_PREFILL_ROWS;
    return std::max(1, std::min(c.max_seq, rows / c.batch));
}

// Chunk buffers: fp32 residual rows h and Q rows (K and V go straight to
// the cache); the GEMM operands (normed rows / attention output, FFN hidden
// rows) as bf16 hi and lo planes in the fragment layout, rows padded to a
// multiple of 16.
struct PrefillLayout {
    size_t h, xh, xl, q, fh, fl, total;   // byte offsets from the workspace base
};
PrefillLayout prefill_layout(const df_config& c) {
    PrefillLayout P{};
    size_t o = layout(c).total;
    const size_t R = (size_t)c.batch * prefill_chunk(c), R16 = (R + 15) / 16 * 16;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
    P.h = take(R * c.d_model * 4);
    P.xh = take(R16 * c.d_model * 2);
    P.xl = take(R16 * c.d_model * 2);
    P.q = take(R * c.d_model * 4);
    P.fh = take(R16 * (size_t)c.ffn * 2);
    P.fl = take(R16 * (size_t)c.ffn * 2);
    P.total = o;
    return P;
}

// Dual forward: chunks of Tc positions per sequence and both flows, the
// stacked rows [primary 0..R-1 | pad | aux R16..R16+R-1] (R16 = R rounded up
// to 16) in every two-flow buffer.
int forward_chunk(const df_config& c) {
    const int rows = (c.prefill_rows > 0 ? c.prefill_rows : DF_PREFILL_ROWS) / 2;
    return std::max(1, std::min(c.max_seq, rows / c.batch));
}
struct ForwardLayout {
    size_t h, xh, xl, q1, q2, fh, fl, keep, logits;   // fast path (byte offsets)
    size_t pmix, alpha, tok;                        // per-position path
    size_t total;
};
ForwardLayout forward_layout(const df_config& c) {
    ForwardLayout F{};
    size_t o = layout(c).total;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
    if (fast_prefill(c)) {
        const size_t R = (size_t)c.batch * forward_chunk(c), R16 = (R + 15) / 16 * 16, d = c.d_model;
        F.h = take(2 * R16 * d * 4);
        F.xh = take(2 * R16 * d * 2);
        F.xl = take(2 * R16 * d * 2);
        F.q1 = take(R * d * 4);
        F.q2 = take(R * d * 4);
        F.fh = take(2 * R16 * (size_t)c.ffn * 2);
        F.fl = take(2 * R16 * (size_t)c.ffn * 2);
        F.keep = take(R * d * 4);
        F.logits = take(2 * R16 * (size_t)c.vocab * 4);
    } else {
        F.pmix = take((size_t)c.batch * c.vocab * 4);
        F.alpha = take((size_t)c.batch * 4);
        F.tok = take((size_t)c.batch * 4);
    }
    F.total = o;
    return F;
}

int mix_mode_of(const df_config& c, int nflows) {
    return nflows == 1 ? DF_MIX_PRIMARY
           : (c.variant & DF_VARIANT_AUX_OUTPUT) ? DF_MIX_AUX
           : (c.variant & DF_VARIANT_ALPHA_HALF) ? DF_MIX_HALF : DF_MIX_COLLISION;
}

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15) == 0; }

int check_config(const df_config* c) {
    if (!c) return DF_ERR_NULL;
    if (c->dtype != DF_F32 && c->dtype != DF_BF16) return DF_ERR_DTYPE;
    if (c->n_layers < 1 || c->d_model < 1 || c->n_heads < 1 || c->vocab < 1 || c->batch < 1 ||
        c->max_seq < 1 || c->n_experts < 0)
        return DF_ERR_SHAPE;
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return DF_ERR_SHAPE;
    if (c->d_model != c->n_heads * c->head_dim || c->d_model > 4096) return DF_ERR_SHAPE;
    if (c->batch > 64) return DF_ERR_SHAPE;
    if (!(c->ln_eps > 0.f) || c->prefill_rows < 0) return DF_ERR_ARG;
    if ((c->variant & ~(DF_VARIANT_NO_COUPLING | DF_VARIANT_AUX_OUTPUT | DF_VARIANT_ALPHA_HALF)) != 0 ||
        ((c->variant & DF_VARIANT_AUX_OUTPUT) && (c->variant & DF_VARIANT_ALPHA_HALF)))
        return DF_ERR_ARG;
    const bool moe = c->n_experts > 0;
    if (c->top_k_aux < 0 || c->top_k_aux > 16 || (!moe && c->top_k_aux != 0) ||
        (moe && c->top_k_aux > c->n_experts))
        return DF_ERR_SHAPE;
    if (moe) {
        if (c->dtype != DF_BF16) return DF_ERR_DTYPE;
        if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts || c->n_experts > 1024) return DF_ERR_SHAPE;
        if (c->expert_ffn < 1 || c->expert_ffn % 256 != 0 || c->n_experts % 16 != 0) return DF_ERR_SHAPE;
    } else {
        if (c->ffn < 1) return DF_ERR_SHAPE;
    }
    if (c->dtype == DF_BF16) {
        if (c->d_model % 256 != 0 || (!moe && c->ffn % 256 != 0) || c->vocab % 16 != 0) return DF_ERR_SHAPE;
    } else {
        if (c->batch > 8 || c->d_model % 4 != 0 || c->ffn % 4 != 0) return DF_ERR_SHAPE;
    }
    return DF_OK;
}

int check_weights(const df_config& c, const df_weights* w) {
    if (!w) return DF_ERR_NULL;
    const void* need[] = {w->tok_emb[0], w->tok_emb[1], w->pos_emb, w->ln1, w->ln2, w->lnf, w->w_qkv, w->w_o,
                          w->cpl_a, w->cpl_b, w->cpl_c, w->w_out};
    for (const void* p : need)
        if (!p) return DF_ERR_NULL;
    for (const void* p : need)
        if (!aligned16(p)) return DF_ERR_ALIGN;
    if (c.n_experts > 0) {
        const void* moe[] = {w->w_router, w->w_exp_up, w->w_exp_down};
        for (const void* p : moe)
            if (!p) return DF_ERR_NULL;
        for (const void* p : moe)
            if (!aligned16(p)) return DF_ERR_ALIGN;
    } else {
        if (!w->w_up || !w->w_down) return DF_ERR_NULL;
        if (!aligned16(w->w_up) || !aligned16(w->w_down)) return DF_ERR_ALIGN;
    }
    return DF_OK;
}

int check_kv(const df_kv* kv) {
    if (!kv || !kv->k || !kv->v || !kv->len) return DF_ERR_NULL;
    if (!aligned16(kv->k) || !aligned16(kv->v) || ((uintptr_t)kv->len & 3)) return DF_ERR_ALIGN;
    return DF_OK;
}

int check_ws(const df_config& c, const void* ws, size_t ws_bytes) {
    if (!ws) return DF_ERR_NULL;
    if ((uintptr_t)ws % kAlign) return DF_ERR_ALIGN;
    if (ws_bytes < layout(c).total) return DF_ERR_WORKSPACE;
    return DF_OK;
}

// --- kernel timing with events --------------------------------------------
struct Timing {
    std::mutex mu;
    int kclass = -1;
    int64_t stride = 1;           // time one launch of the class in every `stride`
    int64_t seen = 0;             // launches of the class since df_timing_enable
    std::vector<hipEvent_t> ev;   // pairs
    size_t used = 0;
};
Timing g_timing;
constexpr size_t kMaxTimed = 65536;

void timing_events(int kclass, hipEvent_t* start, hipEvent_t* stop) {
    *start = nullptr;
    *stop = nullptr;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.kclass != kclass || g_timing.used >= kMaxTimed) return;
    if (g_timing.seen++ % g_timing.stride != 0) return;
    while (g_timing.ev.size() < 2 * (g_timing.used + 1)) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        g_timing.ev.push_back(e);
    }
    *start = g_timing.ev[2 * g_timing.used];
    *stop = g_timing.ev[2 * g_timing.used + 1];
    ++g_timing.used;
}

struct Step {
    const df_config& c;
    const df_weights& w;
    const df_kv& kv;
    char* ws;
    WsLayout L;
    hipStream_t s;

    template <typename P> P* at(size_t off) const { return reinterpret_cast<P*>(ws + off); }

    // One step over all layers; head: run the LM head and mixture head.
    int run(const int32_t* tok, int tok_stride, int nflows, const float* router_logits, float* logits,
            float* p_mix, float* alpha, int32_t* next_tok, int32_t* expert_ids, bool head) {
        const size_t es = elem_size(c.dtype);
        const int B = c.batch, d = c.d_model, L_ = c.n_layers;
        const bool moe = c.n_experts > 0;
        int32_t* status = at<int32_t>(L.status);
        float* h = at<float>(L.h);
        float* xd = at<float>(L.xd);
        float* xo = at<float>(L.xo);
        float* xf = at<float>(L.xf);
        float* q = at<float>(L.q);
        hipError_t e = dfk::embed_ln(c.dtype, w.tok_emb[0], w.tok_emb[1], w.pos_emb, tok, tok_stride, kv.len, B, d,
                                     c.max_seq, c.vocab, nflows, w.ln1, c.ln_eps, h, xd, status, s);
        if (e != hipSuccess) return DF_ERR_HIP;
        const size_t kv_layer = (size_t)B * c.n_heads * c.max_seq * c.head_dim * es;
        const size_t ffn = moe ? (size_t)c.expert_ffn : (size_t)c.ffn;
        // LayerNorms: a residual update leaves per-segment statistics of h;
        // with bf16 storage the next projection normalises h on the fly from
        // them, otherwise ln_apply writes the normalised rows to xd first.
        const bool fused = c.dtype == DF_BF16;
        const bool couple = (c.variant & DF_VARIANT_NO_COUPLING) == 0;   // a, b, c applied
        const int kr = std::max(c.top_k, c.top_k_aux);                   // MoE ranking length
        float* stats = at<float>(L.stats);
        // every projection is k-sliced as for the 2B stacked rows of a dual
        // step, also in a primary-only step: the primary outputs are then
        // summed over the same slices in the same order either way
        const int qkv_slices = dfk::plan_gemv(c.dtype, 3 * d, d, nflows == 2 ? 2 * B : B, 2 * B).S;
        bool pending = false;   // h has fresh statistics whose norm has not been applied
        auto set_x = [&](dfk::GemvArgs& g, const float* gain) {
            if (pending && fused) { g.x = h; g.x_stats = stats; g.x_gain = gain; }
            else { g.x = xd; g.x_stats = nullptr; g.x_gain = nullptr; }
        };
        auto apply_norm = [&](const float* gain) -> bool {   // h -> xd when it is not fused
            if (!pending || fused) return true;
            pending = false;
            return dfk::ln_apply(h, stats, gain, c.ln_eps, B, d, nflows, xd, s) == hipSuccess;
        };
        for (int l = 0; l < L_; ++l) {
            char* kc = reinterpret_cast<char*>(kv.k) + l * kv_layer;
            char* vc = reinterpret_cast<char*>(kv.v) + l * kv_layer;
            const float* g_ln1 = w.ln1 + (size_t)l * d;
            const float* g_ln2 = w.ln2 + (size_t)l * d;
            const float* g_next = (l + 1 < L_) ? w.ln1 + (size_t)(l + 1) * d : w.lnf;
            dfk::GemvArgs g{};
            g.dtype = c.dtype; g.B = B; g.nflows = nflows; g.H = c.n_heads; g.Dh = c.head_dim; g.S_max = c.max_seq;
            g.part = at<float>(L.gpart); g.eps = c.ln_eps; g.slice_rows = 2 * B;
            // Q/K/V projection of LN1(h). bf16: its k-slice partial sums go
            // straight to the attention pass, which sums them, applies the Q
            // coupling and appends the primary K/V; fp32: the projection's
            // epilogue does both
            set_x(g, g_ln1);
            const float* cpl_a = couple ? w.cpl_a + (size_t)l * d : nullptr;
            g.w = reinterpret_cast<const char*>(w.w_qkv) + (size_t)l * 3 * d * d * es;
            g.N = 3 * d; g.K = d; g.epi = fused ? dfk::EPI_PART : dfk::EPI_QKV; g.cpl = cpl_a; g.q_out = q;
            g.kc = kc; g.vc = vc; g.len = kv.len; g.status = status;
            if (dfk::gemv(g, s) != hipSuccess) return DF_ERR_HIP;
            // shared-K/V attention of both queries over positions 0..len[b]
            dfk::AttnArgs a{};
            a.dtype = c.dtype; a.k = kc; a.v = vc; a.B = B; a.H = c.n_heads; a.S_max = c.max_seq; a.Dh = c.head_dim;
            a.q = q; a.a = nullptr; a.nkeys = kv.len; a.nkeys_add = 1; a.nflows = nflows;
            a.part = at<float>(L.part); a.o_rows = xo;
            if (fused) {
                a.qkv_part = g.part; a.qkv_S = qkv_slices; a.a = cpl_a; a.status = status;
            }
            timing_events(0, &a.ev_start, &a.ev_stop);
            if (dfk::attention(a, s) != hipSuccess) return DF_ERR_HIP;
            // output projection + residual (statistics for LN2)
            g.x = xo; g.x_stats = nullptr; g.x_gain = nullptr;
            g.w = reinterpret_cast<const char*>(w.w_o) + (size_t)l * d * d * es;
            g.N = d; g.K = d; g.epi = dfk::EPI_RESID; g.cpl = nullptr; g.h = h; g.stats_out = stats;
            if (dfk::gemv(g, s) != hipSuccess) return DF_ERR_HIP;
            pending = true;
            const float* cb = couple ? w.cpl_b + (size_t)l * ffn : nullptr;
            const float* cc = couple ? w.cpl_c + (size_t)l * d : nullptr;
            if (!moe) {
                if (!apply_norm(g_ln2)) return DF_ERR_HIP;
                set_x(g, g_ln2);
                g.w = reinterpret_cast<const char*>(w.w_up) + (size_t)l * ffn * d * es;
                g.N = (int)ffn; g.K = d; g.epi = dfk::EPI_GELU_B; g.cpl = cb; g.x_out = xf;
                if (dfk::gemv(g, s) != hipSuccess) return DF_ERR_HIP;
                pending = false;
                // down projection + c coupling + residual (statistics for the next norm)
                g.x = xf; g.x_stats = nullptr; g.x_gain = nullptr;
                g.w = reinterpret_cast<const char*>(w.w_down) + (size_t)l * d * ffn * es;
                g.N = d; g.K = (int)ffn; g.epi = dfk::EPI_RESID; g.cpl = cc; g.h = h; g.stats_out = stats;
                if (dfk::gemv(g, s) != hipSuccess) return DF_ERR_HIP;
                pending = true;
                if (!apply_norm(g_next)) return DF_ERR_HIP;
            } else {
                // one kernel per sequence normalises the rows (LN2) and routes them
                const int E = c.n_experts;
                dfk::MoeArgs m{};
                m.dtype = c.dtype; m.h = h; m.stats = stats; m.g_ln = g_ln2;
                m.w_router = reinterpret_cast<const char*>(w.w_router) + (size_t)l * E * d * es;
                m.r1_given = router_logits ? router_logits + (size_t)l * B * E : nullptr;
                m.w_up = reinterpret_cast<const char*>(w.w_exp_up) + (size_t)l * E * ffn * d * es;
                m.w_down = reinterpret_cast<const char*>(w.w_exp_down) + (size_t)l * E * d * ffn * es;
                m.cpl_b = cb; m.cpl_c = cc; m.B = B; m.d = d; m.E = E; m.k = c.top_k; m.Fe = (int)ffn;
                m.ka = c.top_k_aux > 0 ? c.top_k_aux : c.top_k;
                m.nflows = nflows;
                m.ids_out = expert_ids ? expert_ids + (size_t)l * B * kr : nullptr;
                m.x = xd; m.ids = at<int32_t>(L.ids); m.gates = at<float>(L.gates); m.g_rows = at<float>(L.grows);
                m.y_rows = at<float>(L.yrows);
                m.g_next = g_next; m.eps = c.ln_eps; m.x_next = xd;   // next norm fused into the combine
                if (dfk::moe(m, s) != hipSuccess) return DF_ERR_HIP;
                pending = false;
            }
        }
        if (head) {
            float* lg = logits ? logits : at<float>(L.logits);
            dfk::GemvArgs g{};
            g.dtype = c.dtype; g.B = B; g.nflows = nflows; g.w = w.w_out; g.N = c.vocab; g.K = d;
            g.epi = dfk::EPI_STORE; g.out_f32 = lg; g.eps = c.ln_eps;
            g.part = at<float>(L.gpart); g.slice_rows = 2 * B;
            set_x(g, w.lnf);   // final norm
            if (dfk::gemv(g, s) != hipSuccess) return DF_ERR_HIP;
            const int mode = mix_mode_of(c, nflows);
            // the step's last kernel also advances len
            if (dfk::mix_head(lg, B, c.vocab, mode, p_mix, alpha, next_tok, s, kv.len) != hipSuccess)
                return DF_ERR_HIP;
            return DF_OK;
        }
        if (dfk::len_add(kv.len, B, 1, s) != hipSuccess) return DF_ERR_HIP;
        return DF_OK;
    }
};

}  // namespace

extern "C" {

size_t df_workspace_bytes(const df_config* cfg) {
    if (check_config(cfg) != DF_OK) return 0;
    return layout(*cfg).total;
}

int df_decode_step(const df_config* cfg, const df_weights* w, const df_kv* kv, const int32_t* d_tokens,
                   int32_t aux_on, const float* d_router_logits, float* d_logits, float* d_p_mix, float* d_alpha,
                   int32_t* d_next_tok, int32_t* d_expert_ids, void* d_ws, size_t ws_bytes, void* stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_weights(*cfg, w))) return rc;
    if ((rc = check_kv(kv))) return rc;
    if (!d_tokens || !d_p_mix || !d_alpha) return DF_ERR_NULL;
    if (aux_on != 0 && aux_on != 1) return DF_ERR_ARG;
    if (d_router_logits && cfg->n_experts == 0) return DF_ERR_ARG;
    if ((d_logits && !aligned16(d_logits)) || !aligned16(d_p_mix)) return DF_ERR_ALIGN;
    if ((rc = check_ws(*cfg, d_ws, ws_bytes))) return rc;
    Step st{*cfg, *w, *kv, reinterpret_cast<char*>(d_ws), layout(*cfg), reinterpret_cast<hipStream_t>(stream)};
    return st.run(d_tokens, 1, aux_on ? 2 : 1, d_router_logits, d_logits, d_p_mix, d_alpha, d_next_tok,
                  d_expert_ids, true);
}

size_t df_prefill_workspace_bytes(const df_config* cfg) {
    if (check_config(cfg) != DF_OK) return 0;
    return fast_prefill(*cfg) ? prefill_layout(*cfg).total : layout(*cfg).total;
}

int df_prefill_primary(const df_config* cfg, const df_weights* w, const df_kv* kv, const int32_t* d_tokens,
                       int32_t T, void* d_ws, size_t ws_bytes, void* stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_weights(*cfg, w))) return rc;
    if ((rc = check_kv(kv))) return rc;
    if (!d_tokens) return DF_ERR_NULL;
    if (T < 0 || T > cfg->max_seq) return DF_ERR_SHAPE;
    if ((rc = check_ws(*cfg, d_ws, ws_bytes))) return rc;
    if (ws_bytes < df_prefill_workspace_bytes(cfg)) return DF_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const df_config& c = *cfg;
    if (!fast_prefill(c)) {
        Step st{c, *w, *kv, reinterpret_cast<char*>(d_ws), layout(c), s};
        for (int t = 0; t < T; ++t) {
            rc = st.run(d_tokens + t, T, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false);
            if (rc) return rc;
        }
        return DF_OK;
    }
    // Standard causal Transformer over the prompt, chunk by chunk; every
    // layer of a chunk sees the K/V its earlier chunks left in the cache.
    char* ws = reinterpret_cast<char*>(d_ws);
    const PrefillLayout P = prefill_layout(c);
    int32_t* status = reinterpret_cast<int32_t*>(ws + layout(c).status);
    float* h = reinterpret_cast<float*>(ws + P.h);
    float* q = reinterpret_cast<float*>(ws + P.q);
    void* xh = ws + P.xh;
    void* xl = ws + P.xl;
    void* fh = ws + P.fh;
    void* fl = ws + P.fl;
    const int B = c.batch, d = c.d_model, H = c.n_heads, Dh = c.head_dim, F = c.ffn;
    const size_t es = 2;
    const size_t kv_layer = (size_t)B * H * c.max_seq * Dh * es;
    const int Tmax = prefill_chunk(c);
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    auto timed = [&](int kclass, auto&& launch) -> hipError_t {   // the launch takes its own timestamps
        hipEvent_t e0, e1;
        timing_events(kclass, &e0, &e1);
        return launch(e0, e1);
    };
    auto gemm = [&](const void* ah, const void* al, const char* wt, int R, int N, int K, int epi, float* y,
                    const dfk::QkvStore* st = nullptr) {
        return timed(1, [&](hipEvent_t e0, hipEvent_t e1) {
            return dfk::gemm(ah, al, wt, R, N, K, epi, y, fh, fl, s, st, nullptr, e0, e1);
        });
    };
    for (int t0 = 0; t0 < T; t0 += Tmax) {
        const int Tc = std::min(Tmax, T - t0), R = B * Tc;
        if (!ok(dfk::prefill_embed_rows(w->tok_emb[0], w->pos_emb, d_tokens, T, t0, Tc, kv->len, B, d, c.max_seq,
                                        c.vocab, h, status, s)))
            return DF_ERR_HIP;
        for (int l = 0; l < c.n_layers; ++l) {
            char* kc = reinterpret_cast<char*>(kv->k) + l * kv_layer;
            char* vc = reinterpret_cast<char*>(kv->v) + l * kv_layer;
            const char* wqkv = reinterpret_cast<const char*>(w->w_qkv) + (size_t)l * 3 * d * d * es;
            const char* wo = reinterpret_cast<const char*>(w->w_o) + (size_t)l * d * d * es;
            const char* wup = reinterpret_cast<const char*>(w->w_up) + (size_t)l * F * d * es;
            const char* wdn = reinterpret_cast<const char*>(w->w_down) + (size_t)l * d * F * es;
            const dfk::QkvStore st{reinterpret_cast<uint16_t*>(kc), reinterpret_cast<uint16_t*>(vc), kv->len, Tc,
                                   t0, H, Dh, c.max_seq, status};
            if (!ok(dfk::prefill_layer_norm(h, w->ln1 + (size_t)l * d, c.ln_eps, R, d, xh, xl, s)) ||
                !ok(gemm(xh, xl, wqkv, R, 3 * d, d, dfk::GEMM_QKV, q, &st)) ||
                !ok(timed(2, [&](hipEvent_t e0, hipEvent_t e1) {
                    return dfk::prefill_attention(q, B, Tc, t0, kv->len, H, Dh, c.max_seq, kc, vc, xh, xl, s,
                                                  nullptr, nullptr, 0, e0, e1);
                })) ||
                !ok(gemm(xh, xl, wo, R, d, d, dfk::GEMM_RESID, h)) ||
                !ok(dfk::prefill_layer_norm(h, w->ln2 + (size_t)l * d, c.ln_eps, R, d, xh, xl, s)) ||
                !ok(gemm(xh, xl, wup, R, F, d, dfk::GEMM_GELU_SPLIT, nullptr)) ||
                !ok(gemm(fh, fl, wdn, R, d, F, dfk::GEMM_RESID, h)))
                return DF_ERR_HIP;
        }
    }
    return ok(dfk::len_add(kv->len, B, T, s)) ? DF_OK : DF_ERR_HIP;
}

size_t df_forward_workspace_bytes(const df_config* cfg) {
    if (check_config(cfg) != DF_OK) return 0;
    return forward_layout(*cfg).total;
}

int df_forward_dual(const df_config* cfg, const df_weights* w, const df_kv* kv, const int32_t* d_tokens,
                    int32_t T, float* d_logits, float* d_p_mix, float* d_alpha, int32_t* d_next_tok, void* d_ws,
                    size_t ws_bytes, void* stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_weights(*cfg, w))) return rc;
    if ((rc = check_kv(kv))) return rc;
    if (!d_tokens || !d_p_mix || !d_alpha) return DF_ERR_NULL;
    if (T < 0 || T > cfg->max_seq) return DF_ERR_SHAPE;
    if ((d_logits && !aligned16(d_logits)) || !aligned16(d_p_mix)) return DF_ERR_ALIGN;
    if ((rc = check_ws(*cfg, d_ws, ws_bytes))) return rc;
    if (ws_bytes < df_forward_workspace_bytes(cfg)) return DF_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const df_config& c = *cfg;
    char* ws = reinterpret_cast<char*>(d_ws);
    const ForwardLayout F = forward_layout(c);
    const WsLayout L0 = layout(c);
    const int B = c.batch, d = c.d_model, V = c.vocab;
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    if (!fast_prefill(c)) {
        // one dual step per position (the decode-step kernels), each row of
        // outputs copied to its place in the [batch][T] buffers
        Step st{c, *w, *kv, ws, L0, s};
        float* lg = reinterpret_cast<float*>(ws + L0.logits);
        float* pm = reinterpret_cast<float*>(ws + F.pmix);
        float* al = reinterpret_cast<float*>(ws + F.alpha);
        int32_t* tk = reinterpret_cast<int32_t*>(ws + F.tok);
        for (int t = 0; t < T; ++t) {
            rc = st.run(d_tokens + t, T, 2, nullptr, lg, pm, al, d_next_tok ? tk : nullptr, nullptr, true);
            if (rc) return rc;
            const size_t f4 = sizeof(float);
            if (!ok(hipMemcpy2DAsync(d_p_mix + (size_t)t * V, (size_t)T * V * f4, pm, V * f4, V * f4, B,
                                     hipMemcpyDeviceToDevice, s)) ||
                !ok(hipMemcpy2DAsync(d_alpha + t, (size_t)T * f4, al, f4, f4, B, hipMemcpyDeviceToDevice, s)) ||
                (d_next_tok && !ok(hipMemcpy2DAsync(d_next_tok + t, (size_t)T * 4, tk, 4, 4, B,
                                                    hipMemcpyDeviceToDevice, s))) ||
                (d_logits && !ok(hipMemcpy2DAsync(d_logits + (size_t)t * 2 * V, (size_t)T * 2 * V * f4, lg,
                                                  2 * V * f4, 2 * V * f4, B, hipMemcpyDeviceToDevice, s))))
                return DF_ERR_HIP;
        }
        return DF_OK;
    }
    // Both flows through the chunk rows: the primary rows are the prefill's;
    // the aux rows take their query from the shared W_q rows, attend the
    // primary K/V, and get the b / c couplings in the aux GEMM epilogues.
    int32_t* status = reinterpret_cast<int32_t*>(ws + L0.status);
    float* h = reinterpret_cast<float*>(ws + F.h);
    bf16p xh = ws + F.xh, xl = ws + F.xl, fh = ws + F.fh, fl = ws + F.fl;
    float* q1 = reinterpret_cast<float*>(ws + F.q1);
    float* q2 = reinterpret_cast<float*>(ws + F.q2);
    float* keep = reinterpret_cast<float*>(ws + F.keep);
    float* lgt = reinterpret_cast<float*>(ws + F.logits);
    const int H = c.n_heads, Dh = c.head_dim, Fd = c.ffn;
    const bool couple = (c.variant & DF_VARIANT_NO_COUPLING) == 0;
    const size_t es = 2;
    const size_t kv_layer = (size_t)B * H * c.max_seq * Dh * es;
    const int Tmax = forward_chunk(c);
    auto timed = [&](int kclass, auto&& launch) -> hipError_t {   // the launch takes its own timestamps
        hipEvent_t e0, e1;
        timing_events(kclass, &e0, &e1);
        return launch(e0, e1);
    };
    auto gemm = [&](const void* ah, const void* al, const void* wt, int R, int N, int K, int epi, float* y, void* oh,
                    void* ol, const dfk::QkvStore* qs = nullptr, const dfk::GemmCouple* cp = nullptr) {
        return timed(1, [&](hipEvent_t e0, hipEvent_t e1) {
            return dfk::gemm(ah, al, wt, R, N, K, epi, y, oh, ol, s, qs, cp, e0, e1);
        });
    };
    for (int t0 = 0; t0 < T; t0 += Tmax) {
        const int Tc = std::min(Tmax, T - t0), R = B * Tc, R16 = (R + 15) / 16 * 16, R2 = R16 + R;
        const size_t xa = (size_t)R16 * d * es, fa = (size_t)R16 * Fd * es;   // byte offsets of the aux rows
        float* h2 = h + (size_t)R16 * d;
        if (!ok(dfk::prefill_embed_rows(w->tok_emb[0], w->pos_emb, d_tokens, T, t0, Tc, kv->len, B, d, c.max_seq,
                                        V, h, status, s, w->tok_emb[1], R16)))
            return DF_ERR_HIP;
        for (int l = 0; l < c.n_layers; ++l) {
            char* kc = reinterpret_cast<char*>(kv->k) + l * kv_layer;
            char* vc = reinterpret_cast<char*>(kv->v) + l * kv_layer;
            const char* wqkv = reinterpret_cast<const char*>(w->w_qkv) + (size_t)l * 3 * d * d * es;
            const char* wo = reinterpret_cast<const char*>(w->w_o) + (size_t)l * d * d * es;
            const char* wup = reinterpret_cast<const char*>(w->w_up) + (size_t)l * Fd * d * es;
            const char* wdn = reinterpret_cast<const char*>(w->w_down) + (size_t)l * d * Fd * es;
            const dfk::QkvStore st{reinterpret_cast<uint16_t*>(kc), reinterpret_cast<uint16_t*>(vc), kv->len, Tc,
                                   t0, H, Dh, c.max_seq, status};
            const dfk::GemmCouple cb{w->cpl_b + (size_t)l * Fd, reinterpret_cast<const uint16_t*>(fh),
                                     reinterpret_cast<const uint16_t*>(fl), nullptr};
            const dfk::GemmCouple cc{w->cpl_c + (size_t)l * d, nullptr, nullptr, keep};
            if (!ok(dfk::prefill_layer_norm(h, w->ln1 + (size_t)l * d, c.ln_eps, R2, d, xh, xl, s)) ||
                !ok(gemm(xh, xl, wqkv, R, 3 * d, d, dfk::GEMM_QKV, q1, nullptr, nullptr, &st)) ||
                !ok(gemm(xh + xa, xl + xa, wqkv, R, d, d, dfk::GEMM_STORE, q2, nullptr, nullptr)) ||
                !ok(timed(2, [&](hipEvent_t e0, hipEvent_t e1) {
                    return dfk::prefill_attention(q1, B, Tc, t0, kv->len, H, Dh, c.max_seq, kc, vc, xh, xl, s, q2,
                                                  couple ? w->cpl_a + (size_t)l * d : nullptr, R16, e0, e1);
                })) ||
                !ok(gemm(xh, xl, wo, R2, d, d, dfk::GEMM_RESID, h, nullptr, nullptr)) ||
                !ok(dfk::prefill_layer_norm(h, w->ln2 + (size_t)l * d, c.ln_eps, R2, d, xh, xl, s)) ||
                !ok(gemm(xh, xl, wup, R, Fd, d, dfk::GEMM_GELU_SPLIT, nullptr, fh, fl)) ||
                !ok(gemm(xh + xa, xl + xa, wup, R, Fd, d, couple ? dfk::GEMM_GELU_SPLIT_CPL : dfk::GEMM_GELU_SPLIT,
                         nullptr, fh + fa, fl + fa, nullptr, &cb)) ||
                !ok(gemm(fh, fl, wdn, R, d, Fd, couple ? dfk::GEMM_RESID_KEEP : dfk::GEMM_RESID, h, nullptr, nullptr,
                         nullptr, &cc)) ||
                !ok(gemm(fh + fa, fl + fa, wdn, R, d, Fd, couple ? dfk::GEMM_RESID_CPL : dfk::GEMM_RESID, h2, nullptr,
                         nullptr, nullptr, &cc)))
                return DF_ERR_HIP;
        }
        // final norm, the shared LM head over both flows' rows, the mixture per position
        if (!ok(dfk::prefill_layer_norm(h, w->lnf, c.ln_eps, R2, d, xh, xl, s)) ||
            !ok(gemm(xh, xl, w->w_out, R2, V, d, dfk::GEMM_STORE, lgt, nullptr, nullptr)) ||
            !ok(dfk::mix_rows(lgt, lgt + (size_t)R16 * V, R, V, mix_mode_of(c, 2), Tc, T, t0, d_logits, d_p_mix,
                              d_alpha, d_next_tok, s)))
            return DF_ERR_HIP;
    }
    return ok(dfk::len_add(kv->len, B, T, s)) ? DF_OK : DF_ERR_HIP;
}

int df_kv_append(const df_config* cfg, const df_kv* kv, int32_t layer, const int32_t* d_pos, const float* d_k,
                 const float* d_v, int32_t* d_status, void* stream) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if ((rc = check_kv(kv))) return rc;
    if (!d_pos || !d_k || !d_v) return DF_ERR_NULL;
    if (layer < 0 || layer >= cfg->n_layers) return DF_ERR_SHAPE;
    const size_t es = elem_size(cfg->dtype);
    const size_t kv_layer = (size_t)cfg->batch * cfg->n_heads * cfg->max_seq * cfg->head_dim * es;
    hipError_t e = dfk::kv_append(cfg->dtype, reinterpret_cast<char*>(kv->k) + layer * kv_layer,
                                  reinterpret_cast<char*>(kv->v) + layer * kv_layer, cfg->batch, cfg->n_heads,
                                  cfg->max_seq, cfg->head_dim, d_pos, d_k, d_v, d_status,
                                  reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? DF_OK : DF_ERR_HIP;
}

int df_mix_head(const float* d_logits, int32_t batch, int32_t vocab, int32_t mode, float* d_p_mix,
                float* d_alpha, int32_t* d_next_tok, void* stream) {
    if (!d_logits || !d_p_mix || !d_alpha) return DF_ERR_NULL;
    if (batch < 1 || vocab < 1) return DF_ERR_SHAPE;
    if (mode < DF_MIX_PRIMARY || mode > DF_MIX_HALF) return DF_ERR_ARG;
    hipError_t e = dfk::mix_head(d_logits, batch, vocab, mode, d_p_mix, d_alpha, d_next_tok,
                                 reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? DF_OK : DF_ERR_HIP;
}

size_t df_attention_workspace_bytes(int32_t batch, int32_t n_heads, int32_t max_seq, int32_t head_dim) {
    if (batch < 1 || n_heads < 1 || max_seq < 1 || (head_dim != 32 && head_dim != 64 && head_dim != 128)) return 0;
    return align_up(dfk::attention_part_floats(batch, n_heads, max_seq, head_dim) * 4);
}

int df_attention_dual(int32_t dtype, const void* d_k, const void* d_v, int32_t batch, int32_t n_heads,
                      int32_t max_seq, int32_t head_dim, const int32_t* d_len, const float* d_q, const float* d_a,
                      float* d_o, float* d_lse, void* d_ws, size_t ws_bytes, void* stream) {
    return dfk::attention_dual_entry(dtype, d_k, d_v, batch, n_heads, max_seq, head_dim, d_len, d_q, d_a, d_o,
                                     d_lse, d_ws, ws_bytes, stream, true);
}

size_t df_stacked_gemv_workspace_bytes(int32_t dtype, int32_t rows, int32_t N, int32_t K) {
    if ((dtype != DF_F32 && dtype != DF_BF16) || rows < 1 || N < 1 || K < 1) return 0;
    if (dtype == DF_BF16 && rows > kStackedRows) {   // tiled GEMM: the rows as hi / lo fragment planes
        if (N % 16 || K % 32) return 0;
        return 2 * align_up((size_t)(rows + 15) / 16 * 16 * K * 2);
    }
    if (rows < 2 || (rows & 1)) return 0;
    if (dtype == DF_BF16 && (K % 256 || N % 16)) return 0;
    if (dtype == DF_F32 && (rows > 16 || K % 4)) return 0;
    const dfk::GemvPlan pl = dfk::plan_gemv(dtype, N, K, rows);
    if (dtype == DF_BF16 && pl.MT == 0) return 0;
    return align_up(pl.part_floats * 4 + kAlign);
}

int df_stacked_gemv(int32_t dtype, const float* d_x, const void* d_w, int32_t rows, int32_t N, int32_t K,
                    float* d_y, void* d_ws, size_t ws_bytes, void* stream) {
    if (dtype != DF_F32 && dtype != DF_BF16) return DF_ERR_DTYPE;
    if (!d_x || !d_w || !d_y || !d_ws) return DF_ERR_NULL;
    const size_t need = df_stacked_gemv_workspace_bytes(dtype, rows, N, K);
    if (need == 0) return DF_ERR_SHAPE;
    if (!aligned16(d_x) || !aligned16(d_w) || !aligned16(d_y) || (uintptr_t)d_ws % kAlign) return DF_ERR_ALIGN;
    if (ws_bytes < need) return DF_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (dtype == DF_BF16 && rows > kStackedRows) {
        char* xh = reinterpret_cast<char*>(d_ws);
        char* xl = xh + need / 2;
        if (dfk::split_rows(d_x, rows, K, xh, xl, s) != hipSuccess) return DF_ERR_HIP;
        return dfk::gemm(xh, xl, d_w, rows, N, K, dfk::GEMM_STORE, d_y, nullptr, nullptr, s) == hipSuccess
                   ? DF_OK
                   : DF_ERR_HIP;
    }
    dfk::GemvArgs g{};
    g.dtype = dtype; g.x = d_x; g.w = d_w; g.N = N; g.K = K; g.B = rows / 2; g.nflows = 2;
    g.epi = dfk::EPI_STORE; g.out_f32 = d_y; g.part = reinterpret_cast<float*>(d_ws);
    return dfk::gemv(g, s) == hipSuccess ? DF_OK : DF_ERR_HIP;
}

int df_pack_weights(int32_t dtype, const void* d_src, void* d_dst, int64_t n_mats, int32_t rows, int32_t cols,
                    void* stream) {
    if (dtype != DF_BF16) return DF_ERR_DTYPE;
    if (!d_src || !d_dst) return DF_ERR_NULL;
    if (n_mats < 1 || n_mats > 65535 || rows < 16 || cols < 32 || rows % 16 || cols % 32) return DF_ERR_SHAPE;
    if (!aligned16(d_src) || !aligned16(d_dst)) return DF_ERR_ALIGN;
    const size_t bytes = (size_t)n_mats * rows * cols * 2;
    const char* a = reinterpret_cast<const char*>(d_src);
    const char* b = reinterpret_cast<const char*>(d_dst);
    if (a < b + bytes && b < a + bytes) return DF_ERR_ARG;   // overlapping buffers
    return dfk::pack_weights(d_src, d_dst, (long)n_mats, rows, cols, reinterpret_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? DF_OK
               : DF_ERR_HIP;
}

int df_device_status(void* d_ws, void* stream, int32_t* status_out) {
    if (!d_ws || !status_out) return DF_ERR_NULL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int32_t v = 0;
    if (hipMemcpyAsync(&v, d_ws, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return DF_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return DF_ERR_HIP;
    const int32_t zero = 0;
    if (hipMemcpyAsync(d_ws, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess) return DF_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return DF_ERR_HIP;
    *status_out = v;
    return DF_OK;
}

const char* df_status_str(int code) {
    switch (code) {
        case DF_OK: return "ok";
        case DF_ERR_NULL: return "a required pointer is NULL";
        case DF_ERR_SHAPE: return "unsupported or inconsistent sizes";
        case DF_ERR_DTYPE: return "unknown or unsupported storage dtype";
        case DF_ERR_ALIGN: return "misaligned pointer";
        case DF_ERR_WORKSPACE: return "workspace too small";
        case DF_ERR_KV_FULL: return "K/V cache full";
        case DF_ERR_HIP: return "HIP launch error";
        case DF_ERR_ARG: return "invalid argument";
    }
    return "unknown status code";
}

int df_timing_enable(int32_t kclass, int32_t stride) {
    if (kclass < 0 || kclass > 2 || stride < 1) return DF_ERR_ARG;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.kclass = kclass;
    g_timing.stride = stride;
    g_timing.seen = 0;
    g_timing.used = 0;
    return DF_OK;
}

int df_timing_read(double* total_ms, int64_t* launches) {
    if (!total_ms || !launches) return DF_ERR_NULL;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    double t = 0.0;
    for (size_t i = 0; i < g_timing.used; ++i) {
        if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess) return DF_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess) return DF_ERR_HIP;
        t += ms;
    }
    *total_ms = t;
    *launches = (int64_t)g_timing.used;
    g_timing.kclass = -1;
    g_timing.used = 0;
    return DF_OK;
}

}  // extern "C"

namespace dfk {

int attention_dual_entry(int dtype, const void* d_k, const void* d_v, int batch, int n_heads, int max_seq,
                         int head_dim, const int32_t* d_len, const float* d_q, const float* d_a, float* d_o,
                         float* d_lse, void* d_ws, size_t ws_bytes, void* stream, bool timed) {
    if (dtype != DF_F32 && dtype != DF_BF16) return DF_ERR_DTYPE;
    if (!d_k || !d_v || !d_len || !d_q || !d_o || !d_lse || !d_ws) return DF_ERR_NULL;
    if (batch < 1 || n_heads < 1 || max_seq < 1 || (head_dim != 32 && head_dim != 64 && head_dim != 128))
        return DF_ERR_SHAPE;
    if (!attention_fits(batch, n_heads)) return DF_ERR_SHAPE;
    if (!aligned16(d_k) || !aligned16(d_v) || !aligned16(d_q) || (d_a && !aligned16(d_a)) ||
        (uintptr_t)d_ws % kAlign)
        return DF_ERR_ALIGN;
    if (ws_bytes < df_attention_workspace_bytes(batch, n_heads, max_seq, head_dim)) return DF_ERR_WORKSPACE;
    AttnArgs a{};
    a.dtype = dtype; a.k = d_k; a.v = d_v; a.B = batch; a.H = n_heads; a.S_max = max_seq; a.Dh = head_dim;
    a.q = d_q; a.a = d_a; a.nkeys = d_len; a.nkeys_add = 0; a.nflows = 2; a.part = reinterpret_cast<float*>(d_ws);
    a.o_f32 = d_o; a.lse = d_lse; a.o_rows = nullptr;
    if (timed) timing_events(0, &a.ev_start, &a.ev_stop);
    return attention(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? DF_OK : DF_ERR_HIP;
}

}  // namespace dfk
