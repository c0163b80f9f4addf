// df_attention_dual_noalloc: the shared-K/V dual-query attention with its
// partial results in a library-owned device array instead of a
// caller-provided workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). The kernels are those of df_attention_dual.
#include <hip/hip_runtime.h>

#include <mutex>

#include "df_internal.h"
#include "../../include/dualflow.h"

namespace {

constexpr size_t kScratchFloats = dfk::kAttnPartFloatsMax;   // 17,040,384 bytes
static_assert(kScratchFloats * 4 == DF_ATTENTION_NOALLOC_SCRATCH_BYTES, "scratch size");

// One copy per GPU the library runs on, held until the process ends. Every
// call on a GPU uses that GPU's copy: calls that overlap on one GPU (on
// different streams, or from several threads) race.
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's copy, looked up once per device
// (hipGetSymbolAddress with that device current); nullptr on failure.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" int df_attention_dual_noalloc(int32_t dtype, const void* d_k, const void* d_v, int32_t batch,
                                         int32_t n_heads, int32_t max_seq, int32_t head_dim, const int32_t* d_len,
                                         const float* d_q, const float* d_a, float* d_o, float* d_lse,
                                         void* stream) {
    if (df_attention_workspace_bytes(batch, n_heads, max_seq, head_dim) > DF_ATTENTION_NOALLOC_SCRATCH_BYTES)
        return DF_ERR_WORKSPACE;
    void* ws = scratch_ptr();
    if (!ws) return DF_ERR_HIP;
    // no kernel timing here: its first use creates event objects
    return dfk::attention_dual_entry(dtype, d_k, d_v, batch, n_heads, max_seq, head_dim, d_len, d_q, d_a, d_o,
                                     d_lse, ws, DF_ATTENTION_NOALLOC_SCRATCH_BYTES, stream, false);
}
