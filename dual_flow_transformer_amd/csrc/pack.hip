// Repacking of row-major bf16 projection matrices into the 16x32 fragment
// layout the stacked-row GEMV and the MoE expert kernels read (each
// wave-wide load of a matrix-core A operand becomes one contiguous 1 KiB
// piece; see mfma_tile.h).
#include "df_device.h"
#include "df_internal.h"

namespace dfk {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One thread per 16-byte piece q = (t * K/32 + kb) * 64 + lane of a matrix:
// it holds row 16t + lane%16, columns 32kb + 8(lane/16) .. +7.
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                   long pieces_per_mat, int cols) {
    const long q = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long mat = blockIdx.y;
    if (q >= pieces_per_mat) return;
    const int lane = (int)(q & 63);
    const long blk = q >> 6;
    const int KB = cols / 32;
    const long t = blk / KB;
    const int kb = (int)(blk - t * KB);
    const long row = t * 16 + (lane & 15);
    const int col = kb * 32 + (lane >> 4) * 8;
    const size_t base = (size_t)mat * pieces_per_mat * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + base + (size_t)row * cols + col);
    *reinterpret_cast<u32x4*>(dst + base + (size_t)q * 8) = v;
}

}  // namespace

hipError_t pack_weights(const void* src, void* dst, long n_mats, int rows, int cols, hipStream_t s) {
    const long pieces = (long)rows * cols / 8;
    if (n_mats < 1 || n_mats > 65535 || pieces < 1) return hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((pieces + 255) / 256), (unsigned)n_mats), dim3(256), 0, s,
                       reinterpret_cast<const bf16_t*>(src), reinterpret_cast<bf16_t*>(dst), pieces, cols);
    return hipGetLastError();
}

}  // namespace dfk
