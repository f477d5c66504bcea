// Top-k weighted combine for gfx950.
//
// What it computes: "AMD GPU ... 7x faster ... efficient MoE with any number
// of experts" (dignews.cc), opening paragraphs -- a token's output is the sum
// of its chosen experts' FFN outputs weighted by their gate values; the
// GC-MoE abstract (zhuanzhiai.com) adds the shared expert, which here is the
// appended column with weight 1.  The sum runs in ascending k in fp32.
// Unpermute-combine reads the same rows from the permuted (padded expert
// order) buffer through the inverse row map written by the permute: the
// TransformerEngine paragraph of the same page names unpermute as the reverse
// of the permute.
//
// A streaming kernel: each thread owns 4 consecutive hidden units of one
// token (8 when the slot rows are bf16), reads the K slot rows with 16-byte
// non-temporal loads (each y_slots row is read exactly once) and writes fp32
// or bf16.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kCombineThreads = 256;

// kMapped: the rows come from the permuted buffer through row_of_slot (a
// row < 0 is a skipped slot); otherwise from y_slots by slot, skipping ids
// outside [0,E).  The arithmetic is the same, so both give the same bits.
// w == nullptr: every weight is 1 (the unweighted sum of a token's rows,
// which is the gradient of the permute).
template <bool kBf16, bool kMapped>
__global__ void __launch_bounds__(kCombineThreads)
combine_kernel(int T, int K, int E, int H, int nchunk, const float* __restrict__ y,
               const float* __restrict__ w, const int32_t* __restrict__ ids, void* __restrict__ out) {
    const int t = blockIdx.x / nchunk;
    const int h = ((blockIdx.x % nchunk) * kCombineThreads + threadIdx.x) * 4;
    if (h >= H) return;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
        const int64_t i = (int64_t)t * K + k;
        int64_t row = i;
        if (kMapped) {
            row = ids[i];
            if (row < 0) continue;
        } else {
            const int e = ids[i];
            if (e < 0 || e >= E) continue;
        }
        const float wk = w ? w[i] : 1.f;
        const f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)(y + row * H + h));
        acc[0] += wk * v[0];
        acc[1] += wk * v[1];
        acc[2] += wk * v[2];
        acc[3] += wk * v[3];
    }
    if (kBf16) {
        const uint32_t lo = (uint32_t)f32_to_bf16_bits(acc[0]) | ((uint32_t)f32_to_bf16_bits(acc[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_bits(acc[2]) | ((uint32_t)f32_to_bf16_bits(acc[3]) << 16);
        // the layer's output is not read again here: non-temporal
        __builtin_nontemporal_store(u32x2_t{lo, hi}, (u32x2_t*)((uint16_t*)out + (int64_t)t * H + h));
    } else {
        *(f32x4_t*)((float*)out + (int64_t)t * H + h) = acc;
    }
}

// Slot rows in bf16: each thread owns 8 consecutive hidden units (one 16-byte
// load per slot row), widens them exactly to fp32 and sums in the order and
// arithmetic of combine_kernel.
template <bool kBf16>
__global__ void __launch_bounds__(kCombineThreads)
combine_bf16_slots_kernel(int T, int K, int E, int H, int nchunk, const uint16_t* __restrict__ y,
                          const float* __restrict__ w, const int32_t* __restrict__ ids, void* __restrict__ out) {
    const int t = blockIdx.x / nchunk;
    const int h = ((blockIdx.x % nchunk) * kCombineThreads + threadIdx.x) * 8;
    if (h >= H) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
        const int64_t i = (int64_t)t * K + k;
        const int e = ids[i];
        if (e < 0 || e >= E) continue;
        const float wk = w[i];
        const i32x4_t v = __builtin_nontemporal_load((const i32x4_t*)(y + i * H + h));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[2 * j] += wk * __uint_as_float((uint32_t)v[j] << 16);
            acc[2 * j + 1] += wk * __uint_as_float((uint32_t)v[j] & 0xFFFF0000u);
        }
    }
    if (kBf16) {
        i32x4_t o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = (int)((uint32_t)f32_to_bf16_bits(acc[2 * j]) | ((uint32_t)f32_to_bf16_bits(acc[2 * j + 1]) << 16));
        __builtin_nontemporal_store(o, (i32x4_t*)((uint16_t*)out + (int64_t)t * H + h));
    } else {
        float* dst = (float*)out + (int64_t)t * H + h;
        *(f32x4_t*)dst = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
        *(f32x4_t*)(dst + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    }
}

template <bool kMapped>
static hipError_t launch_combine_t(int T, int K, int E, int H, const float* y, const float* w,
                                   const int32_t* idx, int out_bf16, void* out, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int nchunk = (H / 4 + kCombineThreads - 1) / kCombineThreads;
    const dim3 grid((unsigned)((int64_t)T * nchunk));
    if (out_bf16)
        hipLaunchKernelGGL((combine_kernel<true, kMapped>), grid, dim3(kCombineThreads), 0, stream, T, K, E,
                           H, nchunk, y, w, idx, out);
    else
        hipLaunchKernelGGL((combine_kernel<false, kMapped>), grid, dim3(kCombineThreads), 0, stream, T, K, E,
                           H, nchunk, y, w, idx, out);
    return hipGetLastError();
}

hipError_t launch_combine(int T, int K, int E, int H, const float* y_slots, const float* w,
                          const int32_t* ids, int out_bf16, void* out, hipStream_t stream) {
    return launch_combine_t<false>(T, K, E, H, y_slots, w, ids, out_bf16, out, stream);
}

hipError_t launch_combine_bf16_slots(int T, int K, int E, int H, const uint16_t* y_slots, const float* w,
                                     const int32_t* ids, int out_bf16, void* out, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int nchunk = (H / 8 + kCombineThreads - 1) / kCombineThreads;
    const dim3 grid((unsigned)((int64_t)T * nchunk));
    if (out_bf16)
        hipLaunchKernelGGL(combine_bf16_slots_kernel<true>, grid, dim3(kCombineThreads), 0, stream, T, K, E, H,
                           nchunk, y_slots, w, ids, out);
    else
        hipLaunchKernelGGL(combine_bf16_slots_kernel<false>, grid, dim3(kCombineThreads), 0, stream, T, K, E, H,
                           nchunk, y_slots, w, ids, out);
    return hipGetLastError();
}

hipError_t launch_unpermute_combine(int T, int K, int H, const float* y_perm, const float* w,
                                    const int32_t* row_of_slot, int out_bf16, void* out, hipStream_t stream) {
    return launch_combine_t<true>(T, K, 0, H, y_perm, w, row_of_slot, out_bf16, out, stream);
}

}  // namespace moe
