// Device twin of the counter-based input generator in gen.c: the same
// function of (seed, stream, index), bit for bit (integer SplitMix64 steps,
// one double multiply, one round to fp32, bf16 round-to-nearest-even).
// It fills device buffers with seeded inputs quickly; it holds none of the
// Dual-Flow arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define G64 0x9E3779B97F4A7C15ULL

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

__device__ __forceinline__ float normal_at(uint64_t key, uint64_t i, double scale) {
    const uint64_t w = mix64(key + (i + 1) * G64);
    const int32_t s = (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) +
                      (int32_t)((w >> 32) & 0xFFFF) + (int32_t)(w >> 48);
    return (float)((double)(s - 131070) * scale);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Stream s (id streams[s]) fills n_per elements at dst + s*pitch.
__global__ void fill_kernel(void* dst, int64_t n_per, int64_t pitch, uint64_t seed, const uint64_t* streams,
                            double scale, int bf16) {
    const int64_t s = blockIdx.y;
    const uint64_t key = mix64(mix64(seed + G64) ^ streams[s]);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_per; i += (int64_t)gridDim.x * blockDim.x) {
        const float v = normal_at(key, (uint64_t)i, scale);
        if (bf16) reinterpret_cast<uint16_t*>(dst)[s * pitch + i] = bf16_rne(v);
        else reinterpret_cast<float*>(dst)[s * pitch + i] = v;
    }
}

extern "C" int synth_dev_normal_streams(void* dst, int64_t n_streams, int64_t n_per, int64_t pitch, uint64_t seed,
                                        const uint64_t* d_streams, double sigma, int bf16, void* stream) {
    if (n_streams <= 0 || n_per <= 0) return 0;
    if (n_streams > 65535) return -1;
    const double scale = sigma * (1.0 / sqrt((65536.0 * 65536.0 - 1.0) / 3.0));
    int64_t bx = (n_per + 255) / 256;
    if (bx > 4096) bx = 4096;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)bx, (unsigned)n_streams), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), dst, n_per, pitch, seed, d_streams, scale, bf16);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
