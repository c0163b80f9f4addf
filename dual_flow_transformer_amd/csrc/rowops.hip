// Row-wise kernels of the decode step: token + position embedding with the
// first LayerNorm, LayerNorm of the stacked residual rows, the explicit K/V
// write, the length update, and the mixture head.
#include "df_device.h"
#include "df_internal.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

constexpr int kRowThreads = 256;
constexpr int kMaxPerThread = 16;   // d <= 4096

// LayerNorm of one row held in registers (x[e] is element tid + e*256, g[e]
// its gain); the normalised row is written in fp32 (projection inputs are not
// rounded).
__device__ void ln_store(const float (&x)[kMaxPerThread], const float (&g)[kMaxPerThread], int d, float eps,
                         float* out, float* red) {
    const int tid = threadIdx.x;
    float s = 0.f;
    #pragma unroll
    for (int e = 0; e < kMaxPerThread; ++e) {
        const int i = tid + e * kRowThreads;
        if (i < d) s += x[e];
    }
    const float mean = df::block_sum(s, red) / (float)d;
    float v = 0.f;
    #pragma unroll
    for (int e = 0; e < kMaxPerThread; ++e) {
        const int i = tid + e * kRowThreads;
        if (i < d) { const float t = x[e] - mean; v = fmaf(t, t, v); }
    }
    const float var = df::block_sum(v, red) / (float)d;
    const float rstd = 1.0f / sqrtf(var + eps);
    #pragma unroll
    for (int e = 0; e < kMaxPerThread; ++e) {
        const int i = tid + e * kRowThreads;
        if (i < d) out[i] = (x[e] - mean) * rstd * g[e];
    }
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void embed_ln_kernel(
    const T* emb0, const T* emb1, const T* pos_emb, const int32_t* tok, int tok_stride,
    const int32_t* len, int d, int S_max, int V, const float* g, float eps, float* h, float* x, int32_t* status) {
    __shared__ float red[16];
    const int b = blockIdx.x, f = blockIdx.y;   // one workgroup per stacked row (grid y: the flows)
    int pos = len[b];
    pos = pos < 0 ? 0 : (pos >= S_max ? S_max - 1 : pos);
    int t = tok[(size_t)b * tok_stride];
    if (t < 0 || t >= V) {          // out-of-range token id: clamp and flag
        if (status && threadIdx.x == 0) status[0] |= 2;
        t = t < 0 ? 0 : V - 1;
    }
    {
        const T* e = (f == 0 ? emb0 : emb1) + (size_t)t * d;
        const T* pe = pos_emb + (size_t)pos * d;
        const size_t row = (size_t)(2 * b + f) * d;
        // all loads first, unconditional (a column past d reads column d - 1
        // and is masked), so they are in flight together
        float xe[kMaxPerThread], xp[kMaxPerThread], gv[kMaxPerThread];
        #pragma unroll
        for (int k = 0; k < kMaxPerThread; ++k) {
            const int i = min((int)threadIdx.x + k * kRowThreads, d - 1);
            xe[k] = df::St<T>::ld(e, i);
            xp[k] = df::St<T>::ld(pe, i);
            gv[k] = g[i];
        }
        float xv[kMaxPerThread];
        #pragma unroll
        for (int k = 0; k < kMaxPerThread; ++k) {
            const int i = threadIdx.x + k * kRowThreads;
            xv[k] = i < d ? xe[k] + xp[k] : 0.f;
            if (i < d) h[row + i] = xv[k];
        }
        ln_store(xv, gv, d, eps, x + row, red);
    }
}

// x[r] = LN(h[r]; g) from the per-segment statistics of h: block (segment,
// sequence), thread per column, both flows.
__global__ __launch_bounds__(kStatSeg) void ln_apply_kernel(const float* h, const float* stats, const float* g,
                                                            float eps, int d, int nflows, float* x) {
    __shared__ float2 s_mr[2];
    const int seg = blockIdx.x, b = blockIdx.y, nseg = stat_segs(d);
    if ((int)threadIdx.x < nflows) {
        const int r = 2 * b + threadIdx.x;
        s_mr[threadIdx.x] = df::row_norm_from_segments(reinterpret_cast<const float2*>(stats) + (size_t)r * nseg,
                                                       nseg, kStatSeg, d, eps);
    }
    __syncthreads();
    const int n = seg * kStatSeg + threadIdx.x;
    if (n >= d) return;
    for (int f = 0; f < nflows; ++f) {
        const size_t i = (size_t)(2 * b + f) * d + n;
        x[i] = (h[i] - s_mr[f].x) * s_mr[f].y * g[n];
    }
}

template <typename T>
__global__ void kv_append_kernel(T* k, T* v, int H, int S_max, int Dh, const int32_t* pos,
                                 const float* dk, const float* dv, int32_t* status) {
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int p = pos[b];
    if (p < 0 || p >= S_max) {
        if (status && threadIdx.x == 0) status[0] |= 1;
        return;
    }
    for (int i = threadIdx.x; i < Dh; i += blockDim.x) {
        const size_t dst = ((size_t)bh * S_max + p) * Dh + i;
        df::St<T>::st(k, dst, dk[(size_t)bh * Dh + i]);
        df::St<T>::st(v, dst, dv[(size_t)bh * Dh + i]);
    }
}

__global__ void len_add_kernel(int32_t* len, int B, int inc) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) len[b] += inc;
}

// Mixture head: one block of 1024 threads per output row. mode: DF_MIX_*.
// Input row i: l1 = m.l1 + i * m.stride, l2 = m.l2 + i * m.stride; output
// row i, or with m.Tc > 0 the row (i / Tc) * T + t0 + i % Tc of [B][T]
// outputs (chunk row i = b * Tc + t); m.logits_out, if set, receives both
// logit rows there ([row][2][V]).
struct MixRows {
    const float* l1;
    const float* l2;
    size_t stride;
    int Tc, T, t0;
    float* logits_out;
    int32_t* len_inc;   // if set: len_inc[row] += 1 once the row is done (the step's last kernel)
};

// NPT > 0: the row's logits are read once into registers (NPT per thread and
// flow, V <= 1024 NPT) and every pass runs from there; NPT == 0: each pass
// reads them again (any V). Both visit logit v = tid + 1024 j in increasing
// j, so their sums, and so their results, are the same bit for bit.
template <int NPT>
__global__ __launch_bounds__(1024) void mix_head_kernel(MixRows m, int V, int mode, float* p_mix, float* alpha,
                                                        int32_t* next_tok) {
    constexpr int NR = NPT > 0 ? NPT : 1;
    const int aux_on = mode != DF_MIX_PRIMARY;
    __shared__ float red[16];
    __shared__ float bv[16];
    __shared__ int bi[16];
    const int i = blockIdx.x;
    const float* l1 = m.l1 + (size_t)i * m.stride;
    const float* l2 = m.l2 + (size_t)i * m.stride;
    const int b = m.Tc > 0 ? (i / m.Tc) * m.T + m.t0 + i % m.Tc : i;
    float x1[NR], x2[NR];
    if constexpr (NPT > 0) {
        #pragma unroll
        for (int j = 0; j < NPT; ++j) {
            const int v = min((int)threadIdx.x + 1024 * j, V - 1);
            x1[j] = l1[v];
            x2[j] = aux_on ? l2[v] : 0.f;   // the aux row is not read in DF_MIX_PRIMARY
        }
    }
    // logit v of flow f: from the registers or from memory
    auto L1 = [&](int j, int v) { if constexpr (NPT > 0) return x1[j]; else return l1[v]; };
    auto L2 = [&](int j, int v) { if constexpr (NPT > 0) return x2[j]; else return l2[v]; };
    const int nj = NPT > 0 ? NPT : (V + 1023) / 1024;
    if (m.logits_out) {
        float* lo = m.logits_out + (size_t)b * 2 * V;
        for (int j = 0; j < nj; ++j) {
            const int v = threadIdx.x + 1024 * j;
            if (v >= V) break;
            lo[v] = L1(j, v);
            lo[V + v] = L2(j, v);
        }
    }
    float mx1 = -INFINITY, mx2 = -INFINITY;
    #pragma unroll
    for (int j = 0; j < nj; ++j) {
        const int v = threadIdx.x + 1024 * j;
        if (v >= V) break;
        mx1 = fmaxf(mx1, L1(j, v));
        if (aux_on) mx2 = fmaxf(mx2, L2(j, v));
    }
    mx1 = df::block_max(mx1, red);
    if (aux_on) mx2 = df::block_max(mx2, red);
    // exponentials, kept in place of the register-resident logits for the
    // output pass (the memory path computes them again there)
    auto E1 = [&](int j, int v) { return __builtin_amdgcn_exp2f((L1(j, v) - mx1) * df::kLog2e); };
    auto E2 = [&](int j, int v) { return __builtin_amdgcn_exp2f((L2(j, v) - mx2) * df::kLog2e); };
    float s1 = 0.f, c1 = 0.f, s2 = 0.f;
    #pragma unroll
    for (int j = 0; j < nj; ++j) {
        const int v = threadIdx.x + 1024 * j;
        if (v >= V) break;
        const float e1 = E1(j, v);
        s1 += e1;
        c1 = fmaf(e1, e1, c1);
        const float e2 = aux_on ? E2(j, v) : 0.f;
        s2 += e2;
        if constexpr (NPT > 0) {
            x1[j] = e1;
            x2[j] = e2;
        }
    }
    s1 = df::block_sum(s1, red);
    c1 = df::block_sum(c1, red);
    if (aux_on) s2 = df::block_sum(s2, red);
    float a = 1.f;
    if (mode == DF_MIX_COLLISION) a = fminf(1.f, fmaxf(0.5f, c1 / (s1 * s1)));
    else if (mode == DF_MIX_HALF) a = fminf(1.f, 0.5f * (1.f + c1 / (s1 * s1)));
    else if (mode == DF_MIX_AUX) a = 0.f;
    const float w1 = a / s1;
    const float w2 = aux_on ? (1.f - a) / s2 : 0.f;
    float best = -1.f;
    int besti = 0x7fffffff;
    float* out = p_mix + (size_t)b * V;
    #pragma unroll
    for (int j = 0; j < nj; ++j) {
        const int v = threadIdx.x + 1024 * j;
        if (v >= V) break;
        float p;
        if constexpr (NPT > 0) {
            p = x1[j] * w1;
            if (aux_on) p = fmaf(x2[j], w2, p);
        } else {
            p = E1(j, v) * w1;
            if (aux_on) p = fmaf(E2(j, v), w2, p);
        }
        out[v] = p;
        if (p > best) { best = p; besti = v; }
    }
    // argmax: larger value wins, equal values take the lower index
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(besti, o, 64);
        if (ov > best || (ov == best && oi < besti)) { best = ov; besti = oi; }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { bv[w] = best; bi[w] = besti; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float bb = bv[0];
        int ii = bi[0];
        for (int k = 1; k < (int)(blockDim.x >> 6); ++k)
            if (bv[k] > bb || (bv[k] == bb && bi[k] < ii)) { bb = bv[k]; ii = bi[k]; }
        if (next_tok) next_tok[b] = ii;
        alpha[b] = a;
        if (m.len_inc) m.len_inc[b] += 1;
    }
}

// Rows through the mixture head, the register-resident kernel when V allows.
hipError_t launch_mix(const MixRows& m, int R, int V, int mode, float* p_mix, float* alpha, int32_t* next_tok,
                      hipStream_t s) {
    (void)hipGetLastError();
    const dim3 g(R), t(1024);
    if (V <= 4 * 1024) hipLaunchKernelGGL(mix_head_kernel<4>, g, t, 0, s, m, V, mode, p_mix, alpha, next_tok);
    else if (V <= 8 * 1024) hipLaunchKernelGGL(mix_head_kernel<8>, g, t, 0, s, m, V, mode, p_mix, alpha, next_tok);
    else if (V <= 16 * 1024) hipLaunchKernelGGL(mix_head_kernel<16>, g, t, 0, s, m, V, mode, p_mix, alpha, next_tok);
    else if (V <= 32 * 1024) hipLaunchKernelGGL(mix_head_kernel<32>, g, t, 0, s, m, V, mode, p_mix, alpha, next_tok);
    else hipLaunchKernelGGL(mix_head_kernel<0>, g, t, 0, s, m, V, mode, p_mix, alpha, next_tok);
    return hipGetLastError();
}

}  // namespace

hipError_t mix_head(const float* logits, int B, int V, int mode, float* p_mix, float* alpha,
                    int32_t* next_tok, hipStream_t s, int32_t* len_inc) {
    const MixRows m{logits, logits + V, (size_t)2 * V, 0, 0, 0, nullptr, len_inc};
    return launch_mix(m, B, V, mode, p_mix, alpha, next_tok, s);
}

hipError_t mix_rows(const float* l1, const float* l2, int R, int V, int mode, int Tc, int T, int t0,
                    float* logits_out, float* p_mix, float* alpha, int32_t* next_tok, hipStream_t s) {
    const MixRows m{l1, l2, (size_t)V, Tc, T, t0, logits_out, nullptr};
    return launch_mix(m, R, V, mode, p_mix, alpha, next_tok, s);
}

hipError_t kv_append(int dtype, void* k, void* v, int B, int H, int S_max, int Dh, const int32_t* pos,
                     const float* dk, const float* dv, int32_t* status, hipStream_t s) {
    const int threads = Dh < 64 ? 64 : Dh;
    (void)hipGetLastError();
    if (dtype == DF_BF16)
        hipLaunchKernelGGL(kv_append_kernel<bf16_t>, dim3(B * H), dim3(threads), 0, s, (bf16_t*)k, (bf16_t*)v,
                           H, S_max, Dh, pos, dk, dv, status);
    else
        hipLaunchKernelGGL(kv_append_kernel<float>, dim3(B * H), dim3(threads), 0, s, (float*)k, (float*)v,
                           H, S_max, Dh, pos, dk, dv, status);
    return hipGetLastError();
}

hipError_t len_add(int32_t* len, int B, int inc, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(len_add_kernel, dim3((B + 63) / 64), dim3(64), 0, s, len, B, inc);
    return hipGetLastError();
}

hipError_t embed_ln(int dtype, const void* emb0, const void* emb1, const void* pos_emb, const int32_t* tok,
                    int tok_stride, const int32_t* len, int B, int d, int S_max, int V, int nflows, const float* g,
                    float eps, float* h, void* x, int32_t* status, hipStream_t s) {
    (void)hipGetLastError();
    if (dtype == DF_BF16)
        hipLaunchKernelGGL(embed_ln_kernel<bf16_t>, dim3(B, nflows), dim3(kRowThreads), 0, s, (const bf16_t*)emb0,
                           (const bf16_t*)emb1, (const bf16_t*)pos_emb, tok, tok_stride, len, d, S_max, V, g,
                           eps, h, (float*)x, status);
    else
        hipLaunchKernelGGL(embed_ln_kernel<float>, dim3(B, nflows), dim3(kRowThreads), 0, s, (const float*)emb0,
                           (const float*)emb1, (const float*)pos_emb, tok, tok_stride, len, d, S_max, V, g,
                           eps, h, (float*)x, status);
    return hipGetLastError();
}

hipError_t ln_apply(const float* h, const float* stats, const float* g, float eps, int B, int d, int nflows,
                    float* x, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(ln_apply_kernel, dim3(stat_segs(d), B), dim3(kStatSeg), 0, s, h, stats, g, eps, d, nflows, x);
    return hipGetLastError();
}


}  // namespace dfk
