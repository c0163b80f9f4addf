// Device-side helpers shared by the kernels of the dual-flow decode step:
// storage-type loads and stores, bf16 rounding, wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;   // bf16 bit pattern

namespace df {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// Low / high bf16 of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two fp32 -> packed bf16 pair (a in the low half), round to nearest even.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Four fp32 values split into bf16 hi = rne(x) and lo = rne(x - hi) parts
// (packed pairs); hi + lo is within 2^-17 |x| of x.
__device__ __forceinline__ void split_hi_lo(const float4& v, uint2& hi, uint2& lo) {
    hi.x = pack_bf16x2(v.x, v.y);
    hi.y = pack_bf16x2(v.z, v.w);
    lo.x = pack_bf16x2(v.x - bf16_lo(hi.x), v.y - bf16_hi(hi.x));
    lo.y = pack_bf16x2(v.z - bf16_lo(hi.y), v.w - bf16_hi(hi.y));
}

// Storage-type traits: load as fp32, store with rounding to the storage type.
template <typename T> struct St;
template <> struct St<float> {
    static __device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
    static __device__ __forceinline__ float rnd(float v) { return v; }
};
template <> struct St<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void st(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
    static __device__ __forceinline__ float rnd(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// DPP move within rows of 16 lanes (all source lanes valid for these controls).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within 16

// Sum over aligned groups of N lanes (N in 4, 8, 16, 32, 64); every lane of a
// group ends with the same (bitwise) total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<kQuadSwap1>(x);
    x += dpp<kQuadSwap2>(x);
    if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
    if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

// Wave-wide sum and maximum, every lane ending with the same value: exchanges
// within rows of 16 lanes by DPP, then two cross-row shuffles.
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<kQuadSwap1>(x));
    x = fmaxf(x, dpp<kQuadSwap2>(x));
    x = fmaxf(x, dpp<kRowHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
}

// Block-wide sum (blockDim.x a multiple of 64, <= 1024); result to all threads.
__device__ __forceinline__ float block_sum(float x, float* red /* >= 16 floats */) {
    x = wave_sum(x);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i) t += red[i];
    return t;
}
__device__ __forceinline__ float block_max(float x, float* red) {
    x = wave_max(x);
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    float t = red[0];
    for (int i = 1; i < nw; ++i) t = fmaxf(t, red[i]);
    return t;
}

// Mean and 1/sqrt(var + eps) of a row of d values from the (mean, M2) pairs
// of its nseg consecutive segments of seg_len values (the last one possibly
// shorter), by Chan et al.'s pairwise combination of partial moments.
__device__ __forceinline__ float2 row_norm_from_segments(const float2* st, int nseg, int seg_len, int d,
                                                         float eps) {
    float mean = 0.f;
    for (int i = 0; i < nseg; ++i) mean += (float)min(seg_len, d - i * seg_len) * st[i].x;
    mean /= (float)d;
    float m2 = 0.f;
    for (int i = 0; i < nseg; ++i) {
        const float dm = st[i].x - mean;
        m2 += st[i].y + (float)min(seg_len, d - i * seg_len) * dm * dm;
    }
    return make_float2(mean, 1.0f / sqrtf(m2 / (float)d + eps));
}

}  // namespace df
