// kda_state.hip -- state copy used by the prefill entry point when T = 0:
// S_T = S0, or zeros when there is no initial state.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

__global__ void __launch_bounds__(256)
state_copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, size_t n4)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        dst[i] = src ? src[i] : f32x4{0.f, 0.f, 0.f, 0.f};
}

hipError_t launch_state_copy(const float* S0, float* S_T, long long heads, hipStream_t stream)
{
    const size_t n4 = (size_t)heads * (128 * 128 / 4);
    size_t blocks = (n4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const f32x4*>(S0), reinterpret_cast<f32x4*>(S_T), n4);
    return hipGetLastError();
}

}  // namespace kda
