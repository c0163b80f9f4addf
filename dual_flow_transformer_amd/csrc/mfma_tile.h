// Skinny-GEMM building blocks on gfx950 bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16), shared by the stacked-row GEMV and the MoE
// expert kernels.
//
// Operand layout of one 16x16x32 product D = A B (A: 16 x 32, B: 32 x 16):
// lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16] as
// eight bf16 each, and receives D[4*(l/16) + r][l%16] in register r.
// Here A is a 16-row tile of a weight matrix and B the transposed
// activation rows, so D[i][j] = partial sum of weight row i with stacked
// row j.
//
// Weight fragment layout (bf16 [N][K], N % 16 == 0, K % 32 == 0): the A
// operand of 16-row tile t and 32-column block kb is stored as 64
// consecutive 16-byte pieces in lane order,
//   element (n, k) at ((n/16 * K/32 + k/32) * 64 + ((k%32)/8) * 16 + n%16) * 8 + k%8,
// so a wave-wide load of one operand is one contiguous 1 KiB piece and the
// k-blocks of a tile follow each other.
#pragma once

#include "df_device.h"

namespace dfk {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int RT = 2;           // 16-row weight tiles per workgroup
constexpr int ROWS = 16 * RT;   // weight rows per workgroup

// Eight fp32 activations as two bf16 octets, hi = rne(x), lo = rne(x - hi):
// hi + lo equals x to within 2^-17 |x|.
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
    const float4 v0 = *reinterpret_cast<const float4*>(x);
    const float4 v1 = *reinterpret_cast<const float4*>(x + 4);
    const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t h[4], l[4];
    #pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16_t h0 = df::f32_to_bf16(f[2 * i]), h1 = df::f32_to_bf16(f[2 * i + 1]);
        const bf16_t l0 = df::f32_to_bf16(f[2 * i] - df::bf16_to_f32(h0));
        const bf16_t l1 = df::f32_to_bf16(f[2 * i + 1] - df::bf16_to_f32(h1));
        h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    hi = (u32x4){h[0], h[1], h[2], h[3]};
    lo = (u32x4){l[0], l[1], l[2], l[3]};
}

// Offset of element (r, k) of a [*][K] matrix in the fragment layout.
__device__ __forceinline__ size_t frag_off(int r, int k, int K) {
    return ((size_t)((r >> 4) * (K >> 5) + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (r & 15)) * 8 + (k & 7);
}

// Lane's base of 16-row tile t16 in the fragment layout (k-block 0).
__device__ __forceinline__ const bf16_t* frag_tile(const bf16_t* w, int t16, int K, int lane) {
    return w + ((size_t)t16 * (K / 32) * 64 + lane) * 8;
}

// Stream k in [kbeg, kend) (multiple of 32*KU) through MFMAs for RT weight
// tiles (lane bases from frag_tile) against the first `mtiles` activation
// tiles (wave-uniform). The fp32 activation rows enter as bf16 hi and lo
// parts into the same accumulator.
template <int MT, int KU>
__device__ __forceinline__ void stream_k(const bf16_t* const (&wrow)[RT], const float* const (&xrow)[MT],
                                         int mtiles, int kbeg, int kend, f32x4 (&acc)[RT][MT]) {
    for (int k = kbeg; k < kend; k += 32 * KU) {
        u32x4 a[RT][KU], bh[MT][KU], bl[MT][KU];
        #pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            #pragma unroll
            for (int ku = 0; ku < KU; ++ku)
                a[rt][ku] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(wrow[rt] + (size_t)(k / 32 + ku) * 512));
        #pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (mt < mtiles) {
                #pragma unroll
                for (int ku = 0; ku < KU; ++ku) split8(xrow[mt] + k + 32 * ku, bh[mt][ku], bl[mt][ku]);
            }
        #pragma unroll
        for (int ku = 0; ku < KU; ++ku)
            #pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                #pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    if (mt < mtiles) {
                        const bf16x8 av = __builtin_bit_cast(bf16x8, a[rt][ku]);
                        acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av, __builtin_bit_cast(bf16x8, bh[mt][ku]), acc[rt][mt], 0, 0, 0);
                        acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av, __builtin_bit_cast(bf16x8, bl[mt][ku]), acc[rt][mt], 0, 0, 0);
                    }
    }
}

template <int MT>
__device__ __forceinline__ void zero(f32x4 (&acc)[RT][MT]) {
    #pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        #pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// Per-wave accumulators to LDS: red[w][rt][mt][r][lane].
template <int MT>
__device__ __forceinline__ void to_lds(float* red, int wv, int lane, const f32x4 (&acc)[RT][MT]) {
    #pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        #pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            #pragma unroll
            for (int r = 0; r < 4; ++r) red[(((wv * RT + rt) * MT + mt) * 4 + r) * 64 + lane] = acc[rt][mt][r];
}

// Sum over the NW waves (in wave order) of output (weight row nl of the
// workgroup, stacked row m).
template <int MT>
__device__ __forceinline__ float lds_sum(const float* red, int NW, int nl, int m) {
    const int rt = nl >> 4, i = nl & 15, mt = m >> 4, j = m & 15;
    const int idx = ((rt * MT + mt) * 4 + (i & 3)) * 64 + j + 16 * (i >> 2);
    float s = 0.f;
    for (int w = 0; w < NW; ++w) s += red[(size_t)w * RT * MT * 256 + idx];
    return s;
}

// Allow `bytes` of dynamic LDS for kernel `fn` (needed above 64 KiB).
inline hipError_t allow_lds(const void* fn, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

inline int floor_pow2(int x) {
    int r = 1;
    while (r * 2 <= x) r *= 2;
    return r;
}

// Waves per workgroup: about `target` waves over the grid, at most 16, K
// divisible into equal 32*KU-multiples per wave, LDS within 128 KiB.
inline int pick_waves(int n_wg, int K, int MT, int KU, int target) {
    int nw = floor_pow2(target / (n_wg > 0 ? n_wg : 1) > 0 ? target / (n_wg > 0 ? n_wg : 1) : 1);
    if (nw > 16) nw = 16;
    if (nw > 64 / MT) nw = 64 / MT;
    while (nw > 1 && (K % (nw * 32 * KU)) != 0) nw >>= 1;
    return nw;
}

}  // namespace tile
}  // namespace dfk
