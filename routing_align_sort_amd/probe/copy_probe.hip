// Plain streaming kernels of known traffic, used only to calibrate the
// profiler's HBM byte counters and to measure the HBM bandwidth a simple
// kernel reaches on this device.  Not part of the MoE layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

// Reads `n` 16-byte chunks once and writes them once (ordinary loads/stores).
__global__ void __launch_bounds__(256) copy_probe_kernel(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

// Reads `n` 16-byte chunks once; writes one word per workgroup (an xor of
// everything read, so the loads cannot be dropped).
__global__ void __launch_bounds__(256) read_probe_kernel(const uint4* __restrict__ src,
                                                         uint32_t* __restrict__ out, int64_t n) {
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < 256; ++t) r ^= red[t];
        out[blockIdx.x] = r;
    }
}

extern "C" int moe_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16) return 1;
    const int64_t n = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(copy_probe_kernel, dim3(4096), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       (const uint4*)src, (uint4*)dst, n);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// out must hold 4096 words.
extern "C" int moe_probe_read(const void* src, void* out, size_t bytes, void* stream) {
    if (!src || !out || bytes % 16) return 1;
    const int64_t n = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(read_probe_kernel, dim3(4096), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       (const uint4*)src, (uint32_t*)out, n);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
