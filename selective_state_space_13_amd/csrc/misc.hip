// Small helpers: state copy / clear for an empty sequence.
#include "ssd_kernels.h"

namespace ssd {
namespace {

__global__ __launch_bounds__(256) void copy_state_kernel(const float *__restrict__ src,
                                                         float *__restrict__ dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.0f;
}

}  // namespace

// dst[i] = src[i] (or 0 when src is NULL), with a kernel rather than a memset
// or memcpy node so the call can sit inside a captured graph.
hipError_t launch_copy_state(const float *src, float *dst, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    copy_state_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(src, dst, n);
    return hipGetLastError();
}

}  // namespace ssd
