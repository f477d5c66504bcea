// A plain device copy with ordinary 16-byte loads and stores, used only to
// calibrate the HBM byte counters of the profiler (a kernel of known traffic:
// it reads `bytes` once and writes `bytes` once).  Not part of the MoE layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ void __launch_bounds__(256) copy_probe_kernel(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

extern "C" int moe_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16) return 1;
    const int64_t n = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(copy_probe_kernel, dim3(4096), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       (const uint4*)src, (uint4*)dst, n);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
