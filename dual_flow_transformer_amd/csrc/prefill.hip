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
using tile::frag_off;

// h[r] = E_primary[tok[b][t0 + t]] + P[len[b] + t0 + t] (fp32), r = b * Tc + t.
// Token ids outside [0, V) are clamped and flagged (status bit 1).
__global__ __launch_bounds__(256) void prefill_embed(const bf16_t* emb0, const bf16_t* emb1, const bf16_t* pos_emb,
                                                     const int32_t* tok, int T, int t0, int Tc, const int32_t* len,
                                                     int d, int S_max, int V, int R16, float* h, int32_t* status) {
    const int r = blockIdx.x, b = r / Tc, t = r - b * Tc;
    const bf16_t* emb = blockIdx.y ? emb1 : emb0;       // flow blockIdx.y, rows at flow * R16 + r
    h += (size_t)blockIdx.y * R16 * d;
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

// LN(h[r]; g) for R rows of width d as hi / lo fragment planes: one wave
// per row (four rows per block), each lane up to eight runs of eight
// columns held in registers, wave-level reductions only.
constexpr int LN_RUNS = 8;   // d <= 64 lanes * 8 runs * 8 columns
__global__ __launch_bounds__(256) void prefill_ln(const float* h, const float* g, float eps, int R, int d,
                                                  bf16_t* xh, bf16_t* xl) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R) return;
    const float* hr = h + (size_t)r * d;
    const int nrun = d >> 3;
    float4 v[LN_RUNS][2];
    float s = 0.f;
    #pragma unroll
    for (int e = 0; e < LN_RUNS; ++e) {
        const int c = lane + 64 * e;
        if (c < nrun) {
            v[e][0] = *reinterpret_cast<const float4*>(hr + 8 * c);
            v[e][1] = *reinterpret_cast<const float4*>(hr + 8 * c + 4);
        } else {
            v[e][0] = v[e][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        s += (v[e][0].x + v[e][0].y + v[e][0].z + v[e][0].w) + (v[e][1].x + v[e][1].y + v[e][1].z + v[e][1].w);
    }
    const float mean = df::wave_sum(s) / (float)d;
    float q = 0.f;
    #pragma unroll
    for (int e = 0; e < LN_RUNS; ++e) {
        if (lane + 64 * e >= nrun) continue;
        #pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float4 t = v[e][u];
            q = fmaf(t.x - mean, t.x - mean, q);
            q = fmaf(t.y - mean, t.y - mean, q);
            q = fmaf(t.z - mean, t.z - mean, q);
            q = fmaf(t.w - mean, t.w - mean, q);
        }
    }
    const float rstd = 1.0f / sqrtf(df::wave_sum(q) / (float)d + eps);
    #pragma unroll
    for (int e = 0; e < LN_RUNS; ++e) {
        const int c = lane + 64 * e;
        if (c >= nrun) continue;
        const int k = 8 * c;
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

// Causal attention of a chunk's queries over the cache (positions 0 .. own
// position): workgroup (128 queries, head h, sequence b), wave w takes 32
// queries as two 16-query tiles. Per block of 64 keys, staged in LDS for
// the four waves (the next block already in flight in registers):
// S^T = K Q^T on the matrix cores (K rows from LDS, Q as bf16 hi/lo parts
// in registers), online softmax per query in the log2 domain, then
// O^T += V^T P^T. The order of the key reduction is free, so k-slot
// 8 g + j of the product covers key 4 g + (j % 4) of the even (j < 4) or
// odd (j >= 4) 16-key tile: the slots each lane holds after the score
// product. P thus enters the matrix cores from registers (bf16 hi/lo
// parts), and V^T is laid out in LDS in the same key order. Waves whose
// queries all precede a key block skip it. fp32 accumulation; the output
// rows leave as hi / lo fragment planes, the operand form of the next GEMM.
constexpr int ADH = 128;
constexpr int AKB = 64;          // keys per block
constexpr int AQW = 32;          // queries per wave
constexpr int AQG = 4 * AQW;     // queries per workgroup
constexpr int KSP = ADH + 8;     // K row pitch in LDS (bf16)
constexpr int VSP = AKB + 8;     // V^T row pitch

// Column of key j (0..63 within a block) in the V^T rows: keys 4 g .. 4 g + 3
// of 16-key tile 2 c + o sit at 32 c + 8 g + 4 o.
__device__ __forceinline__ int vt_col(int j) {
    const int c = j >> 5, o = (j >> 4) & 1, g = (j >> 2) & 3;
    return c * 32 + g * 8 + o * 4 + (j & 3);
}

struct AttnRows {
    const float* q1;    // [R][H * Dh] primary queries
    const float* q2;    // [R][H * Dh] aux raw queries (two flows) or NULL
    const float* a;     // [H * Dh] query coupling (Q2 = Q2raw + a * Q1) or NULL
    int nflows;         // 1: prefill; 2: dual forward (flow f output rows at f * R16 + r)
    int R16;
};

__global__ __launch_bounds__(256) void attn_prefill(AttnRows qs, int Tc, int t0, const int32_t* len, int H,
                                                    int S_max, const bf16_t* kc, const bf16_t* vc, float scale_log2,
                                                    bf16_t* oh, bf16_t* ol) {
    __shared__ bf16_t Ks[AKB * KSP];
    __shared__ bf16_t Vt[ADH * VSP];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // heaviest query blocks first: workgroups are dispatched with z slowest,
    // so the blocks of the last positions (the most keys) go out first and
    // the light ones fill in at the end
    const int qb = gridDim.z - 1 - blockIdx.z, h = blockIdx.x, b = blockIdx.y;
    const int d = H * ADH;
    const int pos0 = len[b] + t0;                            // position of chunk row t = 0
    // one flow: 128 positions per workgroup, 32 per wave; two flows: 64
    // positions, waves 0-1 take the primary queries and waves 2-3 the aux
    // queries of the same positions, sharing every staged key block
    const int QG = AQG / qs.nflows, flow = qs.nflows == 2 ? wv >> 1 : 0;
    const int tw0 = qb * QG + (qs.nflows == 2 ? (wv & 1) : wv) * AQW;   // first query (chunk row) of this wave
    const int wave_last = tw0 < Tc ? pos0 + min(Tc - 1, tw0 + AQW - 1) : -1;
    const int last_key = min(pos0 + min(Tc, qb * QG + QG) - 1, S_max - 1);
    const size_t head = ((size_t)b * H + h) * S_max * ADH;

    // the wave's queries as bf16 hi/lo B operands, scaled by log2(e)/sqrt(Dh)
    int t_q[2], qpos[2];
    bf16x8 qh[2][4], ql[2][4];
    #pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        t_q[qt] = tw0 + qt * 16 + li;
        const int tq = min(t_q[qt], Tc - 1);
        qpos[qt] = pos0 + tq;
        const size_t qo = (size_t)(b * Tc + tq) * d + h * ADH;
        const float* qr = (flow ? qs.q2 : qs.q1) + qo;
        #pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float4 a = *reinterpret_cast<const float4*>(qr + ks * 32 + lg * 8);
            float4 c = *reinterpret_cast<const float4*>(qr + ks * 32 + lg * 8 + 4);
            if (flow && qs.a) {   // Q2 = Q2raw + a * Q1
                const int e = h * ADH + ks * 32 + lg * 8;
                const float4 a0 = *reinterpret_cast<const float4*>(qs.a + e);
                const float4 a1 = *reinterpret_cast<const float4*>(qs.a + e + 4);
                const float4 p0 = *reinterpret_cast<const float4*>(qs.q1 + qo + ks * 32 + lg * 8);
                const float4 p1 = *reinterpret_cast<const float4*>(qs.q1 + qo + ks * 32 + lg * 8 + 4);
                a = make_float4(fmaf(a0.x, p0.x, a.x), fmaf(a0.y, p0.y, a.y), fmaf(a0.z, p0.z, a.z),
                                fmaf(a0.w, p0.w, a.w));
                c = make_float4(fmaf(a1.x, p1.x, c.x), fmaf(a1.y, p1.y, c.y), fmaf(a1.z, p1.z, c.z),
                                fmaf(a1.w, p1.w, c.w));
            }
            uint2 h0, l0, h1, l1;
            df::split_hi_lo(make_float4(a.x * scale_log2, a.y * scale_log2, a.z * scale_log2, a.w * scale_log2),
                            h0, l0);
            df::split_hi_lo(make_float4(c.x * scale_log2, c.y * scale_log2, c.z * scale_log2, c.w * scale_log2),
                            h1, l1);
            qh[qt][ks] = __builtin_bit_cast(bf16x8, (u32x4){h0.x, h0.y, h1.x, h1.y});
            ql[qt][ks] = __builtin_bit_cast(bf16x8, (u32x4){l0.x, l0.y, l1.x, l1.y});
        }
    }
    f32x4 oacc[2][8];
    #pragma unroll
    for (int qt = 0; qt < 2; ++qt)
        #pragma unroll
        for (int i = 0; i < 8; ++i) oacc[qt][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m[2] = {-1e30f, -1e30f}, l[2] = {0.f, 0.f};

    // staging: K as 4 pieces of 8 dims per thread (rows of the block), V as
    // 4 consecutive keys x 8 dims per thread (written transposed)
    const int kc8 = tid & 15, kg = tid & 15, vc8 = tid >> 4;
    u32x4 kr[4], vr[4];
    auto fetch = [&](int k0) {
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kk = min(k0 + ((tid + 256 * j) >> 4), last_key);
            kr[j] = *reinterpret_cast<const u32x4*>(kc + head + (size_t)kk * ADH + kc8 * 8);
        }
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = min(k0 + 4 * kg + i, last_key);
            vr[i] = *reinterpret_cast<const u32x4*>(vc + head + (size_t)kk * ADH + vc8 * 8);
        }
    };
    auto stash = [&]() {
        #pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x4*>(&Ks[((tid + 256 * j) >> 4) * KSP + kc8 * 8]) = kr[j];
        const int col = vt_col(4 * kg);
        #pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1, sh = (e & 1) * 16;
            const uint32_t x0 = (vr[0][w] >> sh) & 0xffffu, x1 = (vr[1][w] >> sh) & 0xffffu;
            const uint32_t x2 = (vr[2][w] >> sh) & 0xffffu, x3 = (vr[3][w] >> sh) & 0xffffu;
            *reinterpret_cast<uint2*>(&Vt[(vc8 * 8 + e) * VSP + col]) = make_uint2(x0 | (x1 << 16), x2 | (x3 << 16));
        }
    };

    if (last_key >= 0) fetch(0);
    for (int k0 = 0; k0 <= last_key; k0 += AKB) {
        __syncthreads();                 // every wave is done with the previous block
        stash();
        __syncthreads();
        fetch(min(k0 + AKB, last_key));  // next block (clamped: always a valid address)
        if (k0 > wave_last) continue;    // all of this wave's queries precede the block
        f32x4 s[2][4];
        #pragma unroll
        for (int qt = 0; qt < 2; ++qt)
            #pragma unroll
            for (int kt = 0; kt < 4; ++kt) s[qt][kt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        #pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            #pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(&Ks[(kt * 16 + li) * KSP + ks * 32 + lg * 8]));
                #pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    s[qt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[qt][ks], s[qt][kt], 0, 0, 0);
                    s[qt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[qt][ks], s[qt][kt], 0, 0, 0);
                }
            }
        const bool diag = k0 + AKB - 1 > pos0 + tw0;   // a key of the block may follow a query of the wave
        bf16x8 ph[2][2], pl[2][2];
        #pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            float mb = -INFINITY;
            #pragma unroll
            for (int kt = 0; kt < 4; ++kt)
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (diag && k0 + kt * 16 + 4 * lg + r > qpos[qt]) s[qt][kt][r] = -INFINITY;
                    mb = fmaxf(mb, s[qt][kt][r]);
                }
            mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
            mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
            const float mn = fmaxf(m[qt], mb);
            const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn);
            m[qt] = mn;
            l[qt] *= alpha;
            #pragma unroll
            for (int i = 0; i < 8; ++i) oacc[qt][i] *= alpha;
            #pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
                const f32x4 sa = s[qt][2 * g2], sb = s[qt][2 * g2 + 1];
                const float4 pa = make_float4(__builtin_amdgcn_exp2f(sa[0] - mn), __builtin_amdgcn_exp2f(sa[1] - mn),
                                              __builtin_amdgcn_exp2f(sa[2] - mn), __builtin_amdgcn_exp2f(sa[3] - mn));
                const float4 pb = make_float4(__builtin_amdgcn_exp2f(sb[0] - mn), __builtin_amdgcn_exp2f(sb[1] - mn),
                                              __builtin_amdgcn_exp2f(sb[2] - mn), __builtin_amdgcn_exp2f(sb[3] - mn));
                l[qt] += (pa.x + pa.y + pa.z + pa.w) + (pb.x + pb.y + pb.z + pb.w);
                uint2 ha, la, hb, lb;
                df::split_hi_lo(pa, ha, la);
                df::split_hi_lo(pb, hb, lb);
                ph[qt][g2] = __builtin_bit_cast(bf16x8, (u32x4){ha.x, ha.y, hb.x, hb.y});
                pl[qt][g2] = __builtin_bit_cast(bf16x8, (u32x4){la.x, la.y, lb.x, lb.y});
            }
        }
        #pragma unroll
        for (int g2 = 0; g2 < 2; ++g2)
            #pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(&Vt[(dt * 16 + li) * VSP + g2 * 32 + 8 * lg]));
                #pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ph[qt][g2], oacc[qt][dt], 0, 0, 0);
                    oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[qt][g2], oacc[qt][dt], 0, 0, 0);
                }
            }
    }
    #pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        float lt = l[qt];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        if (t_q[qt] >= Tc) continue;
        const float inv = 1.0f / lt;
        const int row = flow * qs.R16 + b * Tc + t_q[qt];
        #pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const float4 v = make_float4(oacc[qt][dt][0] * inv, oacc[qt][dt][1] * inv, oacc[qt][dt][2] * inv,
                                         oacc[qt][dt][3] * inv);
            uint2 hv, lv;
            df::split_hi_lo(v, hv, lv);
            const size_t o = frag_off(row, h * ADH + dt * 16 + 4 * lg, d);
            *reinterpret_cast<uint2*>(oh + o) = hv;
            *reinterpret_cast<uint2*>(ol + o) = lv;
        }
    }
}

}  // namespace

hipError_t prefill_embed_rows(const void* emb, const void* pos_emb, const int32_t* tok, int T, int t0, int Tc,
                              const int32_t* len, int B, int d, int S_max, int V, float* h, int32_t* status,
                              hipStream_t s, const void* emb_aux, int R16) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(prefill_embed, dim3(B * Tc, emb_aux ? 2 : 1), dim3(256), 0, s,
                       reinterpret_cast<const bf16_t*>(emb), reinterpret_cast<const bf16_t*>(emb_aux),
                       reinterpret_cast<const bf16_t*>(pos_emb), tok, T, t0, Tc, len, d, S_max, V, R16, h, status);
    return hipGetLastError();
}

hipError_t prefill_layer_norm(const float* h, const float* g, float eps, int R, int d, void* xh, void* xl,
                              hipStream_t s) {
    if (d > 64 * LN_RUNS * 8 || d % 32) return hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(prefill_ln, dim3((R + 3) / 4), dim3(256), 0, s, h, g, eps, R, d,
                       reinterpret_cast<bf16_t*>(xh), reinterpret_cast<bf16_t*>(xl));
    return hipGetLastError();
}

hipError_t prefill_attention(const float* q, int B, int Tc, int t0, const int32_t* len, int H, int Dh, int S_max,
                             const void* kc, const void* vc, void* oh, void* ol, hipStream_t s, const float* q2,
                             const float* a, int R16, hipEvent_t ev_start, hipEvent_t ev_stop) {
    if (Dh != ADH) return hipErrorInvalidValue;
    const AttnRows qs{q, q2, a, q2 ? 2 : 1, R16};
    const int QG = AQG / qs.nflows;
    (void)hipGetLastError();
    const bf16_t* kcb = reinterpret_cast<const bf16_t*>(kc);
    const bf16_t* vcb = reinterpret_cast<const bf16_t*>(vc);
    float scale_log2 = df::kLog2e / sqrtf((float)Dh);
    bf16_t* ohb = reinterpret_cast<bf16_t*>(oh);
    bf16_t* olb = reinterpret_cast<bf16_t*>(ol);
    void* args[] = {(void*)&qs, &Tc, &t0, (void*)&len, &H, &S_max, (void*)&kcb, (void*)&vcb, &scale_log2, &ohb, &olb};
    return launch_timed(reinterpret_cast<const void*>(&attn_prefill), dim3(H, B, (Tc + QG - 1) / QG), dim3(256), args,
                        0, s, ev_start, ev_stop);
}

}  // namespace dfk
