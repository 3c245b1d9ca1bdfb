// Dropout keep mask of one head, written out as bytes: a test aid that lets the
// caller compare the device generator with an independent one. It calls the
// same philox_word0 as the attention kernels. The backward pass regenerates
// this pattern instead of storing it (emergent.sh glossary "Flash Attention",
// "Key Components of Flash Attention").
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

__global__ __launch_bounds__(256) void dropout_mask_kernel(uint8_t* mask, int N, uint32_t b,
                                                           uint32_t h, uint32_t thr, PhiloxKey key) {
    const int i = blockIdx.y;
    for (int j = blockIdx.x * 256 + threadIdx.x; j < N; j += gridDim.x * 256) {
        const uint32_t w = philox_word0(b, h, (uint32_t)i, (uint32_t)j, key);
        mask[(size_t)i * N + j] = w >= thr ? 1 : 0;
    }
}

}  // namespace

hipError_t launch_dropout_mask(uint8_t* mask, int B, int H, int N, int b, int h, float p,
                               uint64_t seed, hipStream_t stream) {
    (void)B;
    (void)H;
    const PhiloxKey key{(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    const dim3 grid((unsigned)min((N + 255) / 256, 64), (unsigned)N);
    hipLaunchKernelGGL(dropout_mask_kernel, grid, dim3(256), 0, stream, mask, N, (uint32_t)b,
                       (uint32_t)h, dropout_threshold(p), key);
    return hipGetLastError();
}

}  // namespace fa
