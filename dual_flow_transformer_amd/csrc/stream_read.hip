// df_stream_read: a plain streaming read of device memory in the launch
// shape of the decode attention pass (one 4-wave workgroup per compute unit;
// each wave reads one contiguous share with 16-byte non-temporal loads, 16
// per lane in flight, as the attention pass keeps 8 K and 8 V rows per lane
// in flight). Its only arithmetic is an XOR of the words it reads, so its
// duration is the read rate the attention pass, which reads every K/V byte
// once, can at best reach on the same device; at small sizes it also gives
// the fixed cost of one launch.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/dualflow.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kInFlight = 16;   // 16-byte loads per lane per round
constexpr int kMaxDevices = 64;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16, size_t share,
                                                          uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const unsigned w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const size_t lo = min(n16, (size_t)w * share), hi = min(n16, lo + share);
    u32x4 acc = (u32x4){0u, 0u, 0u, 0u};
    for (size_t i = lo; i < hi; i += 64 * kInFlight) {
        u32x4 r[kInFlight];
        // past the end of the share: the last word is read again and not
        // XORed (a load under a branch would serialise the rounds)
        #pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const size_t j = i + (size_t)u * 64 + lane;
            r[u] = __builtin_nontemporal_load(src + (j < hi ? j : hi - 1));
        }
        #pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const size_t j = i + (size_t)u * 64 + lane;
            const u32x4 z = (u32x4){0u, 0u, 0u, 0u};
            acc ^= (j < hi) ? r[u] : z;
        }
    }
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    #pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
    if (lane == 0) out[w] = x;
}

// 4 waves per compute unit of the current device (cached per device); 0 on failure.
int read_waves() {
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return 0;
    }
    if (dev < kMaxDevices && cached[dev].load()) return cached[dev].load();
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return 0;
    }
    if (dev < kMaxDevices) cached[dev].store(4 * cus);
    return 4 * cus;
}

}  // namespace

extern "C" int df_stream_read(const void* d_src, size_t bytes, uint32_t* d_out, void* stream) {
    if (!d_src || !d_out) return DF_ERR_NULL;
    if (((uintptr_t)d_src & 15) || (bytes & 15) || ((uintptr_t)d_out & 3)) return DF_ERR_ALIGN;
    const int waves = read_waves();
    if (waves <= 0) return DF_ERR_HIP;
    if (waves > DF_STREAM_READ_OUT_WORDS) return DF_ERR_SHAPE;
    const size_t n16 = bytes / 16;
    // each wave's share: whole wave-wide loads (1 KiB), the last share shorter
    const size_t share = (n16 + (size_t)waves * 64 - 1) / ((size_t)waves * 64) * 64;
    hipLaunchKernelGGL(stream_read_kernel, dim3(waves / 4), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4*>(d_src), n16, share, d_out);
    return hipGetLastError() == hipSuccess ? DF_OK : DF_ERR_HIP;
}
