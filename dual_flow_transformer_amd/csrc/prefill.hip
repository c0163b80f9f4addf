// Kernels of the compute-bound primary prefill: the primary flow alone over
// the prompt, a standard causal Transformer (gist.science/es/paper/2608.12385,
// "Arquitectura Central": the aux flow is skipped in prefill; "Costes de
// Inferencia vs. Entrenamiento": prefill costs exactly a standard
// Transformer). The prompt is processed in chunks of rows r = b * Tc + t
// (sequence b, chunk position t); the projections are the tiled GEMM
// (gemm.hip); here are the row kernels and the causal attention.
#include "df_device.h"
#include "df_internal.h"
#include "mfma_tile.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

using tile::bf16x8;
using tile::f32x4;
using tile::u32x4;

// h[r] = E_primary[tok[b][t0 + t]] + P[len[b] + t0 + t] (fp32), r = b * Tc + t.
// Token ids outside [0, V) are clamped and flagged (status bit 1).
__global__ __launch_bounds__(256) void prefill_embed(const bf16_t* emb, const bf16_t* pos_emb, const int32_t* tok,
                                                     int T, int t0, int Tc, const int32_t* len, int d, int S_max,
                                                     int V, float* h, int32_t* status) {
    const int r = blockIdx.x, b = r / Tc, t = r - b * Tc;
    int id = tok[(size_t)b * T + t0 + t];
    if (id < 0 || id >= V) {
        if (status && threadIdx.x == 0) status[0] |= 2;
        id = id < 0 ? 0 : V - 1;
    }
    int pos = len[b] + t0 + t;
    pos = pos < 0 ? 0 : (pos >= S_max ? S_max - 1 : pos);
    for (int i = threadIdx.x; i < d; i += blockDim.x)
        h[(size_t)r * d + i] = df::bf16_to_f32(emb[(size_t)id * d + i]) + df::bf16_to_f32(pos_emb[(size_t)pos * d + i]);
}

// Offset of element (r, k) in the fragment layout of a [*][K] matrix.
__device__ __forceinline__ size_t frag_off(int r, int k, int K) {
    return ((size_t)((r >> 4) * (K >> 5) + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (r & 15)) * 8 + (k & 7);
}

// LN(h[r]; g) for R rows of width d as hi / lo fragment planes: one block
// per row, each thread up to two runs of eight columns held in registers.
__global__ __launch_bounds__(256) void prefill_ln(const float* h, const float* g, float eps, int d, bf16_t* xh,
                                                  bf16_t* xl) {
    __shared__ float red[16];
    const int r = blockIdx.x;
    const float* hr = h + (size_t)r * d;
    float4 v[2][2];
    float s = 0.f;
    #pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int k = 8 * (threadIdx.x + 256 * e);
        if (k < d) {
            v[e][0] = *reinterpret_cast<const float4*>(hr + k);
            v[e][1] = *reinterpret_cast<const float4*>(hr + k + 4);
        } else {
            v[e][0] = v[e][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        s += (v[e][0].x + v[e][0].y + v[e][0].z + v[e][0].w) + (v[e][1].x + v[e][1].y + v[e][1].z + v[e][1].w);
    }
    const float mean = df::block_sum(s, red) / (float)d;
    float q = 0.f;
    #pragma unroll
    for (int e = 0; e < 2; ++e) {
        if (8 * (threadIdx.x + 256 * e) >= d) continue;
        #pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float4 t = v[e][u];
            q = fmaf(t.x - mean, t.x - mean, q);
            q = fmaf(t.y - mean, t.y - mean, q);
            q = fmaf(t.z - mean, t.z - mean, q);
            q = fmaf(t.w - mean, t.w - mean, q);
        }
    }
    const float rstd = 1.0f / sqrtf(df::block_sum(q, red) / (float)d + eps);
    #pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int k = 8 * (threadIdx.x + 256 * e);
        if (k >= d) continue;
        const float4 g0 = *reinterpret_cast<const float4*>(g + k);
        const float4 g1 = *reinterpret_cast<const float4*>(g + k + 4);
        const float4 a = make_float4((v[e][0].x - mean) * rstd * g0.x, (v[e][0].y - mean) * rstd * g0.y,
                                     (v[e][0].z - mean) * rstd * g0.z, (v[e][0].w - mean) * rstd * g0.w);
        const float4 b = make_float4((v[e][1].x - mean) * rstd * g1.x, (v[e][1].y - mean) * rstd * g1.y,
                                     (v[e][1].z - mean) * rstd * g1.z, (v[e][1].w - mean) * rstd * g1.w);
        uint2 h0, l0, h1, l1;
        df::split_hi_lo(a, h0, l0);
        df::split_hi_lo(b, h1, l1);
        const size_t o = frag_off(r, k, d);
        *reinterpret_cast<u32x4*>(xh + o) = (u32x4){h0.x, h0.y, h1.x, h1.y};
        *reinterpret_cast<u32x4*>(xl + o) = (u32x4){l0.x, l0.y, l1.x, l1.y};
    }
}

// K/V columns of the QKV rows to the cache at position len[b] + t0 + t,
// rounded to bf16; positions at or past S_max are skipped and flagged.
__global__ __launch_bounds__(256) void prefill_kv_store(const float* qkv, int Tc, int t0, const int32_t* len,
                                                        int H, int Dh, int S_max, bf16_t* kc, bf16_t* vc,
                                                        int32_t* status) {
    const int r = blockIdx.x, b = r / Tc, t = r - b * Tc;
    const int d = H * Dh;
    const int pos = len[b] + t0 + t;
    if (pos < 0 || pos >= S_max) {
        if (status && threadIdx.x == 0) status[0] |= 1;
        return;
    }
    const float* row = qkv + (size_t)r * 3 * d;
    for (int i = threadIdx.x; i < 2 * d; i += blockDim.x) {
        const int kv = i / d, j = i - kv * d, hh = j / Dh, e = j - hh * Dh;
        bf16_t* cache = kv == 0 ? kc : vc;
        cache[(((size_t)b * H + hh) * S_max + pos) * Dh + e] = df::f32_to_bf16(row[d + i]);
    }
}

// Causal attention of a chunk's queries over the cache (positions 0 .. own
// position): workgroup (64 queries, head h, sequence b), wave w takes 16
// queries. Per block of 64 keys: S^T = K Q^T on the matrix cores (K from
// LDS, Q as bf16 hi/lo parts in registers), online softmax per query in the
// log2 domain, P (hi/lo parts through LDS) then O^T += V^T P^T with V
// transposed into LDS. fp32 accumulation throughout; the output rows leave
// as hi / lo fragment planes, the operand form of the next GEMM.
constexpr int ADH = 128;
constexpr int AKB = 64;                 // keys per block
constexpr int KSP = ADH + 8;            // K row pitch in LDS
constexpr int VSP = AKB + 8;            // V^T row pitch
constexpr int PSP = AKB + 8;            // P row pitch

__global__ __launch_bounds__(256) void attn_prefill(const float* qkv, int Tc, int t0, const int32_t* len, int H,
                                                    int S_max, const bf16_t* kc, const bf16_t* vc, float scale_log2,
                                                    bf16_t* oh, bf16_t* ol) {
    __shared__ bf16_t Ks[AKB * KSP];
    __shared__ bf16_t Vt[ADH * VSP];
    __shared__ bf16_t Ps[4][2][16 * PSP];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int d = H * ADH;
    const int pos0 = len[b] + t0;                       // position of chunk row t = 0
    const int t_q = qb * 64 + wv * 16 + li;             // this lane's query (column li)
    const bool q_ok = t_q < Tc;
    const int qpos = pos0 + min(t_q, Tc - 1);
    const int last_key = min(pos0 + min(Tc, qb * 64 + 64) - 1, S_max - 1);
    const size_t head = ((size_t)b * H + h) * S_max * ADH;

    // the wave's queries as bf16 hi/lo B operands, scaled by log2(e)/sqrt(Dh)
    bf16x8 qh[4], ql[4];
    {
        const float* qr = qkv + (size_t)(b * Tc + min(t_q, Tc - 1)) * 3 * d + h * ADH;
        #pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const float4 a = *reinterpret_cast<const float4*>(qr + ks * 32 + lg * 8);
            const float4 c = *reinterpret_cast<const float4*>(qr + ks * 32 + lg * 8 + 4);
            const float4 a2 = make_float4(a.x * scale_log2, a.y * scale_log2, a.z * scale_log2, a.w * scale_log2);
            const float4 c2 = make_float4(c.x * scale_log2, c.y * scale_log2, c.z * scale_log2, c.w * scale_log2);
            uint2 h0, l0, h1, l1;
            df::split_hi_lo(a2, h0, l0);
            df::split_hi_lo(c2, h1, l1);
            qh[ks] = __builtin_bit_cast(bf16x8, (u32x4){h0.x, h0.y, h1.x, h1.y});
            ql[ks] = __builtin_bit_cast(bf16x8, (u32x4){l0.x, l0.y, l1.x, l1.y});
        }
    }
    f32x4 oacc[8];
    #pragma unroll
    for (int i = 0; i < 8; ++i) oacc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m = -1e30f, l = 0.f;
    bf16_t* pw_h = Ps[wv][0];
    bf16_t* pw_l = Ps[wv][1];

    for (int k0 = 0; k0 <= last_key; k0 += AKB) {
        __syncthreads();
        // K block [64][128] into LDS rows; V block transposed into [128][64]
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid + j * 256;                // 1024 pieces of 8 elements
            const int key = e >> 4, c8 = e & 15;
            const int kk = min(k0 + key, last_key);
            const u32x4 kv = *reinterpret_cast<const u32x4*>(kc + head + (size_t)kk * ADH + c8 * 8);
            *reinterpret_cast<u32x4*>(&Ks[key * KSP + c8 * 8]) = kv;
            const u32x4 vv = *reinterpret_cast<const u32x4*>(vc + head + (size_t)kk * ADH + c8 * 8);
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                Vt[(c8 * 8 + 2 * q) * VSP + key] = (bf16_t)(vv[q] & 0xffffu);
                Vt[(c8 * 8 + 2 * q + 1) * VSP + key] = (bf16_t)(vv[q] >> 16);
            }
        }
        __syncthreads();
        // scores S^T[key][query] for 4 tiles of 16 keys
        f32x4 s[4];
        #pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            s[kt] = (f32x4){0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(&Ks[(kt * 16 + li) * KSP + ks * 32 + lg * 8]));
                s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[ks], s[kt], 0, 0, 0);
                s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[ks], s[kt], 0, 0, 0);
            }
        }
        // causal mask and the block maximum of this lane's query
        float mb = -INFINITY;
        #pragma unroll
        for (int kt = 0; kt < 4; ++kt)
            #pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = k0 + kt * 16 + 4 * lg + rr;
                if (key > qpos) s[kt][rr] = -INFINITY;
                mb = fmaxf(mb, s[kt][rr]);
            }
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float mn = fmaxf(m, mb);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        l *= alpha;
        #pragma unroll
        for (int i = 0; i < 8; ++i) oacc[i] *= alpha;
        // P = exp2(s - m) as bf16 hi/lo, row li (query), columns = keys
        #pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const float4 pv = make_float4(__builtin_amdgcn_exp2f(s[kt][0] - mn), __builtin_amdgcn_exp2f(s[kt][1] - mn),
                                          __builtin_amdgcn_exp2f(s[kt][2] - mn), __builtin_amdgcn_exp2f(s[kt][3] - mn));
            l += pv.x + pv.y + pv.z + pv.w;
            uint2 ph, pl;
            df::split_hi_lo(pv, ph, pl);
            *reinterpret_cast<uint2*>(&pw_h[li * PSP + kt * 16 + 4 * lg]) = ph;
            *reinterpret_cast<uint2*>(&pw_l[li * PSP + kt * 16 + 4 * lg]) = pl;
        }
        // O^T[dim][query] += V^T[dim][key] P^T[key][query] over 2 groups of 32 keys
        #pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
            const bf16x8 bh = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&pw_h[li * PSP + g2 * 32 + 8 * lg]));
            const bf16x8 bl = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&pw_l[li * PSP + g2 * 32 + 8 * lg]));
            #pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(&Vt[(dt * 16 + li) * VSP + g2 * 32 + 8 * lg]));
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, oacc[dt], 0, 0, 0);
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, oacc[dt], 0, 0, 0);
            }
        }
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!q_ok) return;
    const float inv = 1.0f / l;
    const int row = b * Tc + t_q;
    #pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const float4 v = make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv);
        uint2 hv, lv;
        df::split_hi_lo(v, hv, lv);
        const size_t o = frag_off(row, h * ADH + dt * 16 + 4 * lg, d);
        *reinterpret_cast<uint2*>(oh + o) = hv;
        *reinterpret_cast<uint2*>(ol + o) = lv;
    }
}

}  // namespace

hipError_t prefill_embed_rows(const void* emb, const void* pos_emb, const int32_t* tok, int T, int t0, int Tc,
                              const int32_t* len, int B, int d, int S_max, int V, float* h, int32_t* status,
                              hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(prefill_embed, dim3(B * Tc), dim3(256), 0, s, reinterpret_cast<const bf16_t*>(emb),
                       reinterpret_cast<const bf16_t*>(pos_emb), tok, T, t0, Tc, len, d, S_max, V, h, status);
    return hipGetLastError();
}

hipError_t prefill_layer_norm(const float* h, const float* g, float eps, int R, int d, void* xh, void* xl,
                              hipStream_t s) {
    if (d > 16 * 256 || d % 32) return hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(prefill_ln, dim3(R), dim3(256), 0, s, h, g, eps, d, reinterpret_cast<bf16_t*>(xh),
                       reinterpret_cast<bf16_t*>(xl));
    return hipGetLastError();
}

hipError_t prefill_kv(const float* qkv, int B, int Tc, int t0, const int32_t* len, int H, int Dh, int S_max,
                      void* kc, void* vc, int32_t* status, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(prefill_kv_store, dim3(B * Tc), dim3(256), 0, s, qkv, Tc, t0, len, H, Dh, S_max,
                       reinterpret_cast<bf16_t*>(kc), reinterpret_cast<bf16_t*>(vc), status);
    return hipGetLastError();
}

hipError_t prefill_attention(const float* qkv, int B, int Tc, int t0, const int32_t* len, int H, int Dh, int S_max,
                             const void* kc, const void* vc, void* oh, void* ol, hipStream_t s) {
    if (Dh != ADH) return hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(attn_prefill, dim3((Tc + 63) / 64, H, B), dim3(256), 0, s, qkv, Tc, t0, len, H, S_max,
                       reinterpret_cast<const bf16_t*>(kc), reinterpret_cast<const bf16_t*>(vc),
                       df::kLog2e / sqrtf((float)Dh), reinterpret_cast<bf16_t*>(oh), reinterpret_cast<bf16_t*>(ol));
    return hipGetLastError();
}

}  // namespace dfk
