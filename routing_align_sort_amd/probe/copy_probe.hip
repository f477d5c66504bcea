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

// Reads `n` 16-byte chunks once the way the grouped GEMMs stream their
// weights: every load instruction of a wave reads 1 KB of consecutive bytes
// (64 lanes x 16), each wave keeps 8 of them in flight, the loads are
// non-temporal, and workgroup b walks the b-th contiguous slab.  Writes one
// word per workgroup (an xor of everything read).
typedef unsigned int u32x4_probe_t __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) stream_probe_kernel(const uint4* __restrict__ src,
                                                           uint32_t* __restrict__ out, int64_t n) {
    constexpr int kUnroll = 8;
    constexpr int64_t kStep = 4 * kUnroll * 64;           // chunks per workgroup step
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t slab = (per + kStep - 1) / kStep * kStep;
    const int64_t begin = (int64_t)blockIdx.x * slab;
    const int64_t end = begin + slab < n ? begin + slab : n;
    const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
    uint32_t acc = 0;
    for (int64_t i = begin + (int64_t)w * kUnroll * 64 + lane; i < end; i += kStep) {
        u32x4_probe_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + u * 64;
            v[u] = j < end ? __builtin_nontemporal_load((const u32x4_probe_t*)(src + j)) : u32x4_probe_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
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

// out must hold `blocks` words (blocks <= 65536).
extern "C" int moe_probe_stream(const void* src, void* out, size_t bytes, int blocks, void* stream) {
    if (!src || !out || bytes % 16 || blocks <= 0 || blocks > 65536) return 1;
    const int64_t n = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(stream_probe_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       (const uint4*)src, (uint32_t*)out, n);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Matrix-core throughput with no memory traffic: every wave runs `iters`
// rounds of 8 independent 32x32 MFMA accumulation chains on register
// operands (kind 0: bf16 32x32x16; 1: E4M3 x E4M3, 2: E4M3 x E2M1, 3: E2M1 x
// E2M1, each 32x32x64 with unit scales), then folds the accumulators into one
// word per wave so the work cannot be dropped.
template <int kKind>
__global__ void __launch_bounds__(256) mfma_probe_kernel(float* __restrict__ out, int iters) {
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    f32x16 acc[8];
    for (int c = 0; c < 8; ++c)
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    const int lane = threadIdx.x & 63;
    if constexpr (kKind > 0) {
        constexpr int ta = kKind == 3 ? 4 : 0;
        constexpr int tb = kKind >= 2 ? 4 : 0;
        i32x8 a, b;
        for (int i = 0; i < 8; ++i) { a[i] = 0x38383838 ^ (lane + i); b[i] = 0x30303030 ^ (lane * 3 + i); }
        if (ta == 4) for (int i = 4; i < 8; ++i) a[i] = 0;
        if (tb == 4) for (int i = 4; i < 8; ++i) b[i] = 0;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], ta, tb, 0, 127, 0, 127);
    } else {
        bf16x8 a, b;
        for (int i = 0; i < 8; ++i) { a[i] = (__bf16)(0.001f * (lane + i)); b[i] = (__bf16)(0.002f * (lane - i)); }
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
    for (int c = 0; c < 8; ++c)
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    if (lane == 0) out[blockIdx.x * 4 + threadIdx.x / 64] = s;
}

// FLOPs per launch = blocks * 4 waves * iters * 8 * (2*32*32*K), K = 16 (bf16) or 64.
extern "C" int moe_probe_mfma(int kind, float* out, int blocks, int iters, void* stream) {
    if (!out || blocks <= 0 || iters <= 0) return 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (kind) {
        case 0: hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters); break;
        case 1: hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters); break;
        case 2: hipLaunchKernelGGL(mfma_probe_kernel<2>, dim3(blocks), dim3(256), 0, s, out, iters); break;
        case 3: hipLaunchKernelGGL(mfma_probe_kernel<3>, dim3(blocks), dim3(256), 0, s, out, iters); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
