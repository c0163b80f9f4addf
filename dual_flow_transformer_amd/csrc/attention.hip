// Asymmetric shared-K/V attention for the grouped decode step
// (gist.science/es/paper/2608.12385, "Mecanismos Clave": the aux query Q2,
// coupled to Q1 through a_l, attends the primary K1/V1, so both flows are
// served by one read of each K/V region).
//
// Split-K flash decode with an even split of all keys over the waves of the
// launch (one 4-wave workgroup per compute unit). The keys of the
// (sequence, head) pairs are laid end to end (pair p = b*H + h holds n_b
// keys); wave w of G takes a contiguous key range of KE keys (waves of even
// workgroups) or KO keys (odd workgroups), laid out in wave order, which
// covers one segment of each pair it overlaps, so every wave streams the
// same number of bytes whatever the mix of context lengths. KE = KO =
// ceil(total / G) unless the waves average 2048 keys or more: workgroups are
// dispatched round-robin over the eight XCDs, and in such long launches the
// waves on the odd XCDs were measured (per-wave completion timestamps) to
// finish ~6 % later than those on the even ones, so even-workgroup waves
// take 3 % more keys and odd ones 3 % fewer. The split depends only on the
// key counts, never on timing. The partial result of (wave w, pair p) goes to
// slot w + p (unique: the overlaps form a staircase in (w, p)), and the
// slots of a pair are consecutive. Each 16-byte load of a key row is shared
// by both queries; LPP lanes hold one key row (Dh/LPP elements each), so a
// wave-wide load covers PPW consecutive positions. Every lane group keeps
// its own online-softmax state (running max m, sum l, output o) in the log2
// domain; groups merge at the end of a segment. The combine pass merges
// the segments of a pair in a fixed order: deterministic (no result depends
// on timing).
#include <algorithm>

#include "df_device.h"
#include "df_internal.h"
#include "../../include/dualflow.h"

namespace dfk {
namespace {

struct PartParams {
    const void* k;
    const void* v;
    const float* q;
    const float* a;
    const int32_t* nkeys;
    float* part_o;     // [slots][2][Dh]
    float* part_ml;    // [slots][4]
    long long* seq_tab; // [B + 2]: key offset of sequence b's first pair; [B], [B + 1]: KE, KO
    size_t seq_stride; // elements between sequences in the cache
    int B, H, S_max, nkeys_add, nflows;
    int waves;         // G: waves of the launch
    float scale_log2;  // log2(e) / sqrt(Dh)
    // fused finish of the Q/K/V projection: its k-slice partial sums
    // [qkv_S][qkv_M][3 * H * Dh] (nullptr: q holds finished queries)
    const float* qkv;
    int qkv_S, qkv_M;
    int32_t* status;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T, int EPL>
__device__ __forceinline__ void unpack(const u32x4& r, float (&x)[EPL]) {
    if constexpr (sizeof(T) == 2) {
        x[0] = df::bf16_lo(r[0]); x[1] = df::bf16_hi(r[0]);
        x[2] = df::bf16_lo(r[1]); x[3] = df::bf16_hi(r[1]);
        x[4] = df::bf16_lo(r[2]); x[5] = df::bf16_hi(r[2]);
        x[6] = df::bf16_lo(r[3]); x[7] = df::bf16_hi(r[3]);
    } else {
        x[0] = __uint_as_float(r[0]); x[1] = __uint_as_float(r[1]);
        x[2] = __uint_as_float(r[2]); x[3] = __uint_as_float(r[3]);
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sums over the S k-slices (stride floats apart) of EPL consecutive floats at
// each of the R row pointers. The PPW lane groups of a wave hold the same
// elements, so group g loads slices g, g + PPW, ... (adding them in that
// order; all of them in one round while S <= 2 PPW), and the group sums are
// then added across the groups by xor-shuffles; an addition is commutative,
// so every lane ends with the same bits.
template <int EPL, int R, int PPW>
__device__ __forceinline__ void slice_sum(const float* const (&rp)[R], size_t stride, int S, int g,
                                          float (&y)[R][EPL]) {
    constexpr int SB = 2, C = EPL / 4, LPP = 64 / PPW;
    #pragma unroll
    for (int r = 0; r < R; ++r)
        #pragma unroll
        for (int e = 0; e < EPL; ++e) y[r][e] = 0.f;
    for (int s0 = g; s0 < S; s0 += SB * PPW) {
        float4 t[SB][R][C];
        #pragma unroll
        for (int u = 0; u < SB; ++u) {
            const size_t o = (size_t)min(s0 + u * PPW, S - 1) * stride;
            #pragma unroll
            for (int r = 0; r < R; ++r)
                #pragma unroll
                for (int c = 0; c < C; ++c) t[u][r][c] = *reinterpret_cast<const float4*>(rp[r] + o + 4 * c);
        }
        #pragma unroll
        for (int u = 0; u < SB; ++u) {
            if (s0 + u * PPW >= S) break;
            #pragma unroll
            for (int r = 0; r < R; ++r)
                #pragma unroll
                for (int c = 0; c < C; ++c) {
                    y[r][4 * c] += t[u][r][c].x; y[r][4 * c + 1] += t[u][r][c].y;
                    y[r][4 * c + 2] += t[u][r][c].z; y[r][4 * c + 3] += t[u][r][c].w;
                }
        }
    }
    #pragma unroll
    for (int o = LPP; o < 64; o <<= 1)
        #pragma unroll
        for (int r = 0; r < R; ++r)
            #pragma unroll
            for (int e = 0; e < EPL; ++e) y[r][e] += __shfl_xor(y[r][e], o, 64);
}

// EPL values rounded to the cache type, as one 16-byte word.
template <typename T, int EPL>
__device__ __forceinline__ u32x4 pack_row(const float (&x)[EPL]) {
    if constexpr (sizeof(T) == 2) {
        return (u32x4){df::pack_bf16x2(x[0], x[1]), df::pack_bf16x2(x[2], x[3]), df::pack_bf16x2(x[4], x[5]),
                       df::pack_bf16x2(x[6], x[7])};
    } else {
        return (u32x4){__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    }
}

__device__ __forceinline__ int keys_of(const int32_t* nkeys, int b, int add, int S_max) {
    int n = nkeys[b] + add;
    return n < 0 ? 0 : (n > S_max ? S_max : n);
}

// Keys per wave for a launch of G waves over `total` keys: KE for the four
// waves of an even workgroup, KO for those of an odd one (equal below 2048
// keys per wave). Both are rounded up, so the G ranges cover every key.
constexpr int kLongWaveKeys = 2048;
constexpr int kXcdSkewMilli = 30;
__device__ __forceinline__ void wave_keys(long long total, int G, long long& KE, long long& KO) {
    const long long g = (long long)G * 1000;
    const int skew = total >= (long long)kLongWaveKeys * G ? kXcdSkewMilli : 0;
    KE = max(1LL, (total * (1000 + skew) + g - 1) / g);
    KO = max(1LL, (total * (1000 - skew) + g - 1) / g);
}

// First key of wave w: the waves of workgroup pairs (2i, 2i + 1) cover
// 4 (KE + KO) keys in wave order.
__device__ __forceinline__ long long wave_first_key(int w, long long KE, long long KO) {
    if (KE == KO) return (long long)w * KE;
    const int r = w & 7;
    return (long long)(w >> 3) * 4 * (KE + KO) + (r < 4 ? r * KE : 4 * KE + (r - 4) * KO);
}

// The wave whose key range holds `key`.
__device__ __forceinline__ int wave_of_key(long long key, long long KE, long long KO) {
    if (KE == KO) return (int)(key / KE);   // unskewed: one division
    const long long P = 4 * (KE + KO), q = key / P, r = key - q * P;
    return (int)(8 * q + (r < 4 * KE ? r / KE : 4 + (r - 4 * KE) / KO));
}

// FUSED: the queries (and the new key's K/V) come from the Q/K/V
// projection's k-slice partial sums (p.qkv); otherwise from p.q.
template <typename T, int DH, int U, bool FUSED>
__global__ __launch_bounds__(256) void attn_partial(PartParams p) {
    constexpr int EPL = 16 / (int)sizeof(T);   // elements per 16-byte load
    constexpr int LPP = DH / EPL;              // lanes per key row
    constexpr int PPW = 64 / LPP;              // key rows per wave-wide load
    const int lane = threadIdx.x & 63;
    const int g = lane / LPP, sub = lane - (lane / LPP) * LPP;
    const bool dual = p.nflows == 2;

    // Key offsets of the sequences (lane b holds sequence b): pair (b, h)
    // starts at key off_b + h * n_b of the flattened range.
    const int my_raw = lane < p.B ? p.nkeys[lane] : 0;   // the position of the new key (fused finish)
    const int my_n = lane < p.B ? keys_of(p.nkeys, lane, p.nkeys_add, p.S_max) : 0;
    long long incl = (long long)p.H * my_n;      // inclusive prefix over lanes
    for (int o = 1; o < 64; o <<= 1) {
        const long long t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    const long long my_off = incl - (long long)p.H * my_n;
    const long long total = __shfl(incl, 63, 64);
    const int G = p.waves;
    long long KE, KO;   // keys per wave of an even and of an odd workgroup
    wave_keys(total, G, KE, KO);
    if (blockIdx.x == 0 && threadIdx.x < 64) {   // for the combine pass
        if (lane < p.B) p.seq_tab[lane] = my_off;
        if (lane == 0) { p.seq_tab[p.B] = KE; p.seq_tab[p.B + 1] = KO; }
        if (FUSED && p.status) {   // a new key outside the cache is not written
            const int pos = lane < p.B ? p.nkeys[lane] : 0;
            if (__ballot(pos < 0 || pos >= p.S_max) != 0 && lane == 0) p.status[0] |= 1;
        }
    }

    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long k_begin = wave_first_key(w, KE, KO);
    const long long k_end = min(total, k_begin + ((w & 4) ? KO : KE));
    long long key = k_begin;
    while (key < k_end) {
        // sequence of this key: the last b whose offset <= key (it has
        // keys: a sequence without keys shares its offset with the next)
        const unsigned long long below = __ballot(lane < p.B && my_off <= key);
        const int b = 63 - __builtin_clzll(below);   // lane 0: offset 0 <= key
        const int n = __shfl(my_n, b, 64);
        const long long off_b = __shfl(my_off, b, 64);
        const int h = (int)((key - off_b) / n);
        const long long pair_lo = off_b + (long long)h * n;
        const int start = (int)(key - pair_lo);
        const int end = (int)(min(k_end, pair_lo + n) - pair_lo);
        const int slot = w + b * p.H + h;
        key = pair_lo + end;
        // the new key (fused finish only): position n - 1 = nkeys[b], the
        // last key of the pair, lies in this segment
        constexpr bool fused = FUSED;
        const bool has_new = fused && end == n && __shfl(my_raw, b, 64) == n - 1;
        const size_t n3 = (size_t)3 * p.H * DH;
        const float* qkv_row = fused ? p.qkv + (size_t)(dual ? 2 * b : b) * n3 + h * DH + sub * EPL : nullptr;
        const size_t qkv_stride = (size_t)p.qkv_M * n3;
        const size_t off = (size_t)b * p.seq_stride + (size_t)h * p.S_max * DH + sub * EPL;
        const T* kp = reinterpret_cast<const T*>(p.k) + off;
        const T* vp = reinterpret_cast<const T*>(p.v) + off;
        // keys read from the cache: [start, kend) (the new key, if in this
        // segment, comes from the slice sums); the bounds are the same in
        // every lane and kept as scalars
        const int kend = __builtin_amdgcn_readfirstlane(has_new ? end - 1 : end);
        const int j_start = __builtin_amdgcn_readfirstlane(start);
        // U rows per lane group of K and of V; past kend the last key is
        // read again and masked out of the scores
        auto load_block = [&](int j0, u32x4 (&kr)[U], u32x4 (&vr)[U]) {
            #pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = min(j0 + u * PPW + g, kend - 1);
                kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + (size_t)j * DH));
            }
            #pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = min(j0 + u * PPW + g, kend - 1);
                vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + (size_t)j * DH));
            }
        };
        // the segment's first block is requested before the queries, so the
        // two round trips overlap
        u32x4 kr[U], vr[U];
        if (j_start < kend) load_block(j_start, kr, vr);

        float q1[EPL], q2[EPL], kn[EPL], vn[EPL];   // kn, vn: the new key's K and V (has_new)
        {
            const float* qp = p.q + ((size_t)(b * 2) * p.H + h) * DH + sub * EPL;
            if (fused) {
                // one round of loads: q1, q2raw and, in the segment that
                // holds the new key, its K and V rows
                const float* q2r = dual ? qkv_row + n3 : qkv_row;
                if (has_new) {
                    const float* rp[4] = {qkv_row, q2r, qkv_row + (size_t)p.H * DH, qkv_row + (size_t)2 * p.H * DH};
                    float y[4][EPL];
                    slice_sum<EPL, 4, PPW>(rp, qkv_stride, p.qkv_S, g, y);
                    #pragma unroll
                    for (int e = 0; e < EPL; ++e) { q1[e] = y[0][e]; q2[e] = y[1][e]; kn[e] = y[2][e]; vn[e] = y[3][e]; }
                } else {
                    const float* rp[2] = {qkv_row, q2r};
                    float y[2][EPL];
                    slice_sum<EPL, 2, PPW>(rp, qkv_stride, p.qkv_S, g, y);
                    #pragma unroll
                    for (int e = 0; e < EPL; ++e) { q1[e] = y[0][e]; q2[e] = y[1][e]; }
                }
            } else {
                #pragma unroll
                for (int e = 0; e < EPL; ++e) q1[e] = qp[e];
            }
            if (dual) {
                const float* q2p = qp + (size_t)p.H * DH;
                if (!fused) {
                    #pragma unroll
                    for (int e = 0; e < EPL; ++e) q2[e] = q2p[e];
                }
                if (p.a) {
                    const float* ap = p.a + h * DH + sub * EPL;
                    #pragma unroll
                    for (int e = 0; e < EPL; ++e) q2[e] = fmaf(ap[e], q1[e], q2[e]);
                }
            } else {
                #pragma unroll
                for (int e = 0; e < EPL; ++e) q2[e] = 0.f;
            }
            #pragma unroll
            for (int e = 0; e < EPL; ++e) { q1[e] *= p.scale_log2; q2[e] *= p.scale_log2; }
        }
        float m1 = -1e30f, l1 = 0.f, m2 = -1e30f, l2 = 0.f;
        float o1[EPL], o2[EPL];
        #pragma unroll
        for (int e = 0; e < EPL; ++e) { o1[e] = 0.f; o2[e] = 0.f; }

        if (has_new) {
            // K and V of the primary row (slice sums), rounded to the cache
            // type, written to the cache at the new position by lane group 0,
            // then attended first (lane group 0 starts its state with it)
            const u32x4 kw = pack_row<T, EPL>(kn), vw = pack_row<T, EPL>(vn);
            if (g == 0) {
                *reinterpret_cast<u32x4*>(const_cast<T*>(kp) + (size_t)(n - 1) * DH) = kw;
                *reinterpret_cast<u32x4*>(const_cast<T*>(vp) + (size_t)(n - 1) * DH) = vw;
            }
            unpack<T, EPL>(kw, kn);
            unpack<T, EPL>(vw, vn);
            float a1 = 0.f, a2 = 0.f;
            #pragma unroll
            for (int e = 0; e < EPL; ++e) { a1 = fmaf(q1[e], kn[e], a1); a2 = fmaf(q2[e], kn[e], a2); }
            a1 = df::group_sum<LPP>(a1);
            if (dual) a2 = df::group_sum<LPP>(a2);
            if (g == 0) {
                m1 = a1; l1 = 1.f;
                if (dual) { m2 = a2; l2 = 1.f; }
                #pragma unroll
                for (int e = 0; e < EPL; ++e) { o1[e] = vn[e]; o2[e] = dual ? vn[e] : 0.f; }
            }
        }

        for (int j0 = j_start; j0 < kend;) {
            float s1[U], s2[U];
            #pragma unroll
            for (int u = 0; u < U; ++u) {
                float kk[EPL];
                unpack<T, EPL>(kr[u], kk);
                float a1 = 0.f, a2 = 0.f;
                #pragma unroll
                for (int e = 0; e < EPL; ++e) { a1 = fmaf(q1[e], kk[e], a1); a2 = fmaf(q2[e], kk[e], a2); }
                a1 = df::group_sum<LPP>(a1);
                if (dual) a2 = df::group_sum<LPP>(a2);
                const bool valid = (j0 + u * PPW + g) < kend;
                s1[u] = valid ? a1 : -INFINITY;
                s2[u] = valid ? a2 : -INFINITY;
            }
            float mb1 = s1[0], mb2 = s2[0];
            #pragma unroll
            for (int u = 1; u < U; ++u) { mb1 = fmaxf(mb1, s1[u]); mb2 = fmaxf(mb2, s2[u]); }
            const float mn1 = fmaxf(m1, mb1), mn2 = fmaxf(m2, mb2);
            const float al1 = fast_exp2(m1 - mn1), al2 = fast_exp2(m2 - mn2);
            m1 = mn1; m2 = mn2;
            l1 *= al1; l2 *= al2;
            #pragma unroll
            for (int e = 0; e < EPL; ++e) { o1[e] *= al1; o2[e] *= al2; }
            #pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p1 = fast_exp2(s1[u] - mn1);
                const float p2 = dual ? fast_exp2(s2[u] - mn2) : 0.f;
                l1 += p1; l2 += p2;
                float vv[EPL];
                unpack<T, EPL>(vr[u], vv);
                #pragma unroll
                for (int e = 0; e < EPL; ++e) { o1[e] = fmaf(p1, vv[e], o1[e]); o2[e] = fmaf(p2, vv[e], o2[e]); }
            }
            j0 += PPW * U;
            if (j0 >= kend) break;
            load_block(j0, kr, vr);
        }

        // Merge the PPW lane groups (same dims, different key subsets).
        #pragma unroll
        for (int off2 = LPP; off2 < 64; off2 <<= 1) {
            const float m1o = __shfl_xor(m1, off2, 64), l1o = __shfl_xor(l1, off2, 64);
            const float m2o = __shfl_xor(m2, off2, 64), l2o = __shfl_xor(l2, off2, 64);
            const float mn1 = fmaxf(m1, m1o), mn2 = fmaxf(m2, m2o);
            const float sa1 = fast_exp2(m1 - mn1), sb1 = fast_exp2(m1o - mn1);
            const float sa2 = fast_exp2(m2 - mn2), sb2 = fast_exp2(m2o - mn2);
            l1 = l1 * sa1 + l1o * sb1;
            l2 = l2 * sa2 + l2o * sb2;
            #pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float x1 = __shfl_xor(o1[e], off2, 64), x2 = __shfl_xor(o2[e], off2, 64);
                o1[e] = o1[e] * sa1 + x1 * sb1;
                o2[e] = o2[e] * sa2 + x2 * sb2;
            }
            m1 = mn1; m2 = mn2;
        }
        if (g == 0) {
            float* po = p.part_o + (size_t)slot * 2 * DH + sub * EPL;
            #pragma unroll
            for (int e = 0; e < EPL; ++e) po[e] = o1[e];
            if (dual) {
                #pragma unroll
                for (int e = 0; e < EPL; ++e) po[DH + e] = o2[e];
            }
        }
        if (lane == 0) {
            float* pm = p.part_ml + (size_t)slot * 4;
            pm[0] = m1; pm[1] = l1; pm[2] = m2; pm[3] = l2;
        }
    }
}

struct CombParams {
    const float* part_o;
    const float* part_ml;
    const long long* seq_tab;
    const int32_t* nkeys;
    float* o_f32;
    float* lse;
    float* o_rows;
    int B, H, nflows, S_max, nkeys_add;
};

// One workgroup per (sequence, head): thread (cg, f, d4) merges chunks
// cg, cg + NG, ... of flow f for dims 4*d4 .. 4*d4 + 3 (all loads of a thread
// are independent, so they are in flight together), then the NG chunk
// groups merge in a fixed order through LDS: deterministic.
template <int DH>
__global__ __launch_bounds__(256) void attn_combine(CombParams p) {
    constexpr int D4 = DH / 4, PER = 2 * D4, NG = 256 / PER;   // chunk groups
    __shared__ float s_m[NG][2], s_l[NG][2];
    __shared__ float4 s_o[NG][2][D4];
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
    const int cg = threadIdx.x / PER, r = threadIdx.x - cg * PER;
    const int f = r / D4, d4 = r - f * D4;
    // the waves that covered this pair, and so its consecutive slots
    const long long KE = p.seq_tab[p.B], KO = p.seq_tab[p.B + 1];
    const int n = keys_of(p.nkeys, b, p.nkeys_add, p.S_max);
    if (n == 0) {   // no keys: zero output, LSE -inf (no slot belongs to this pair)
        if (f < p.nflows && cg == 0) {
            const size_t row = (size_t)(2 * b + f) * p.H * DH + (size_t)h * DH + 4 * d4;
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            if (p.o_f32) *reinterpret_cast<float4*>(p.o_f32 + row) = z;
            if (p.o_rows) *reinterpret_cast<float4*>(p.o_rows + row) = z;
            if (p.lse && d4 == 0) p.lse[(size_t)(2 * b + f) * p.H + h] = -INFINITY;
        }
        return;
    }
    const long long lo = p.seq_tab[b] + (long long)h * n;
    const int w0 = wave_of_key(lo, KE, KO), w1 = wave_of_key(lo + n - 1, KE, KO);
    const size_t first = (size_t)w0 + (size_t)b * p.H + h;
    const int C = w1 - w0 + 1;
    float m = -1e30f, l = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (f < p.nflows) {
        for (int c0 = cg; c0 < C; c0 += 4 * NG) {
            float mc[4], lc[4];
            float4 oc[4];
            #pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = min(c0 + u * NG, C - 1);
                mc[u] = p.part_ml[(first + c) * 4 + 2 * f];
                lc[u] = p.part_ml[(first + c) * 4 + 2 * f + 1];
                oc[u] = *reinterpret_cast<const float4*>(p.part_o + ((first + c) * 2 + f) * DH + 4 * d4);
            }
            #pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (c0 + u * NG >= C) break;
                const float mn = fmaxf(m, mc[u]);
                const float sa = __builtin_amdgcn_exp2f(m - mn), sb = __builtin_amdgcn_exp2f(mc[u] - mn);
                l = l * sa + lc[u] * sb;
                o.x = o.x * sa + oc[u].x * sb;
                o.y = o.y * sa + oc[u].y * sb;
                o.z = o.z * sa + oc[u].z * sb;
                o.w = o.w * sa + oc[u].w * sb;
                m = mn;
            }
        }
    }
    if (d4 == 0) { s_m[cg][f] = m; s_l[cg][f] = l; }
    s_o[cg][f][d4] = o;
    __syncthreads();
    if (cg != 0 || f >= p.nflows) return;
    for (int g = 1; g < NG; ++g) {
        const float mo = s_m[g][f], lo = s_l[g][f];
        const float4 oo = s_o[g][f][d4];
        const float mn = fmaxf(m, mo);
        const float sa = __builtin_amdgcn_exp2f(m - mn), sb = __builtin_amdgcn_exp2f(mo - mn);
        l = l * sa + lo * sb;
        o.x = o.x * sa + oo.x * sb;
        o.y = o.y * sa + oo.y * sb;
        o.z = o.z * sa + oo.z * sb;
        o.w = o.w * sa + oo.w * sb;
        m = mn;
    }
    const float inv = 1.0f / l;
    o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
    const size_t row = (size_t)(2 * b + f) * p.H * DH + (size_t)h * DH + 4 * d4;
    if (p.o_f32) *reinterpret_cast<float4*>(p.o_f32 + row) = o;
    if (p.o_rows) *reinterpret_cast<float4*>(p.o_rows + row) = o;
    if (p.lse && d4 == 0) p.lse[(size_t)(2 * b + f) * p.H + h] = (m + __log2f(l)) * df::kLn2;
}

constexpr int kMaxSlots = kAttnMaxSlots;   // partial results per launch at most (workspace bound)
constexpr int kTabFloats = 256;            // sequence table [66] 64-bit, padded
static_assert(kTabFloats + (size_t)kMaxSlots * (4 + 2 * 128) == kAttnPartFloatsMax, "workspace bound");

// Waves of an attn_partial launch on the current device (cached): one
// 4-wave workgroup per compute unit. Measured against two and three per CU
// (the occupancy limit) and 1.5 per CU: equal on the longest contexts, up to
// 8 % faster on the shorter ones, and a whole number per CU keeps the CUs
// evenly loaded.
int launch_waves() {
    static int cached = 0;
    if (cached) return cached;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    cached = cus * 4;
    return cached;
}

template <typename T, int DH>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
    constexpr int U = 8;
    const int waves = launch_waves();
    if (waves + a.B * a.H > kMaxSlots) return hipErrorInvalidValue;
    PartParams p;
    p.k = a.k; p.v = a.v; p.q = a.q; p.a = a.a; p.nkeys = a.nkeys;
    p.seq_tab = reinterpret_cast<long long*>(a.part);
    p.part_ml = a.part + kTabFloats;
    p.part_o = p.part_ml + (size_t)kMaxSlots * 4;
    p.seq_stride = (size_t)a.H * a.S_max * DH;
    p.B = a.B; p.H = a.H; p.S_max = a.S_max; p.nkeys_add = a.nkeys_add; p.nflows = a.nflows;
    p.waves = waves;
    p.scale_log2 = df::kLog2e / sqrtf((float)DH);
    p.qkv = a.qkv_part; p.qkv_S = a.qkv_S; p.qkv_M = a.nflows == 2 ? 2 * a.B : a.B; p.status = a.status;
    if (p.qkv && (a.nkeys_add != 1 || a.qkv_S < 1)) return hipErrorInvalidValue;
    void* args[] = {&p};
    const void* fn = p.qkv ? reinterpret_cast<const void*>(&attn_partial<T, DH, U, true>)
                           : reinterpret_cast<const void*>(&attn_partial<T, DH, U, false>);
    hipError_t e = launch_timed(fn, dim3(waves / 4), dim3(256), args, 0, s, a.ev_start, a.ev_stop);
    if (e != hipSuccess) return e;
    CombParams c;
    c.part_o = p.part_o; c.part_ml = p.part_ml; c.seq_tab = p.seq_tab; c.nkeys = a.nkeys; c.o_f32 = a.o_f32;
    c.lse = a.lse; c.o_rows = a.o_rows; c.B = a.B; c.H = a.H; c.nflows = a.nflows; c.S_max = a.S_max;
    c.nkeys_add = a.nkeys_add;
    hipLaunchKernelGGL((attn_combine<DH>), dim3(a.B * a.H), dim3(256), 0, s, c);
    return hipGetLastError();
}

}  // namespace

bool attention_fits(int B, int H) { return B >= 1 && B <= 64 && H >= 1 && launch_waves() + B * H <= kMaxSlots; }

size_t attention_part_floats(int B, int H, int S_max, int Dh) {
    (void)S_max;
    // sequence table, then ml [kMaxSlots][4], then o [kMaxSlots][2][Dh]
    (void)B; (void)H;
    return kTabFloats + (size_t)kMaxSlots * (4 + 2 * Dh);
}

hipError_t attention(const AttnArgs& a, hipStream_t s) {
    if (a.B > 64) return hipErrorInvalidValue;
    if (a.dtype == DF_BF16) {
        switch (a.Dh) {
            case 32: return launch<bf16_t, 32>(a, s);
            case 64: return launch<bf16_t, 64>(a, s);
            case 128: return launch<bf16_t, 128>(a, s);
        }
    } else {
        switch (a.Dh) {
            case 32: return launch<float, 32>(a, s);
            case 64: return launch<float, 64>(a, s);
            case 128: return launch<float, 128>(a, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace dfk
