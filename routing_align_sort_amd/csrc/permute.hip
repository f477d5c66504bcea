// Permute token rows into Align & Sort's padded expert order, and the inverse
// row map, for gfx950.
//
// What it computes: "AMD GPU ... 7x faster ... efficient MoE with any number
// of experts" (dignews.cc), opening paragraphs, the TransformerEngine
// paragraph and its "MoE Permute example" figure -- a permute step moves the
// rows into expert order and records where each source row went; unpermute
// (in combine.hip) reads them back.  The GC-MoE abstract (zhuanzhiai.com)
// names the token dispatch and the combine around the grouped GEMMs under
// expert parallelism: with the padded expert order every expert's rows are
// contiguous, so each destination GPU's experts form one contiguous range of
// the permuted buffer.
//
//   x_perm[r]      = x[sorted[r] / K]   for sorted[r] < S, else a zero row
//   scale_perm[r]  = x_scale[sorted[r] / K], else 0     (optional)
//   row_of_slot[i] = r with sorted[r] = i; -1 when ids[i] is outside [0,E)
// for rows r below P = num_tokens_post_padded; rows from P to the capacity
// hold no expert's data and are not written (the grid is sized by capacity,
// so P stays on the device).
//
// One wave per row: a lane moves 16 bytes per instruction, a wave 1 KB of the
// row at a time.  The two writers of row_of_slot touch disjoint slots (every
// in-range slot is placed exactly once, out-of-range slots never), so they
// need no ordering.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kPermRowsPerWg = kPermThreads / kWave;

__global__ void __launch_bounds__(kPermThreads)
permute_rows_kernel(const uint8_t* __restrict__ x, int64_t row_bytes, int K, int E, int64_t S, int64_t C,
                    const int32_t* __restrict__ sorted, const int32_t* __restrict__ post_padded,
                    const int32_t* __restrict__ ids,
                    const float* __restrict__ x_scale, uint8_t* __restrict__ x_perm,
                    float* __restrict__ scale_perm, int32_t* __restrict__ row_of_slot) {
    const int lane = lane_id();
    const int64_t g = (int64_t)blockIdx.x * kPermThreads + threadIdx.x;
    if (g < S) {
        const int e = ids[g];
        if (e < 0 || e >= E) row_of_slot[g] = -1;
    }
    const int64_t r = (int64_t)blockIdx.x * kPermRowsPerWg + threadIdx.x / kWave;
    if (r >= C || r >= post_padded[0]) return;
    const int slot = sorted[r];
    const bool placed = slot >= 0 && slot < S;
    const int64_t t = placed ? slot / K : 0;
    if (lane == 0) {
        if (placed) row_of_slot[slot] = (int32_t)r;
        if (scale_perm) scale_perm[r] = placed ? x_scale[t] : 0.f;
    }
    const int64_t nch = row_bytes / 16;
    const uint4* src = (const uint4*)(x + t * row_bytes);
    uint4* dst = (uint4*)(x_perm + r * row_bytes);
    if (placed) {
#pragma unroll 4
        for (int64_t c = lane; c < nch; c += kWave) dst[c] = src[c];
    } else {
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        for (int64_t c = lane; c < nch; c += kWave) dst[c] = z;
    }
}

hipError_t launch_permute_rows(const void* x, int64_t row_bytes, int K, int E, int64_t S, int64_t C,
                               const int32_t* sorted, const int32_t* post_padded, const int32_t* ids,
                               const float* x_scale, void* x_perm, float* scale_perm, int32_t* row_of_slot,
                               hipStream_t stream) {
    if (C == 0) return hipSuccess;
    const int64_t nwg = (C + kPermRowsPerWg - 1) / kPermRowsPerWg;   // also covers the S slots: C >= S
    hipLaunchKernelGGL(permute_rows_kernel, dim3((unsigned)nwg), dim3(kPermThreads), 0, stream,
                       (const uint8_t*)x, row_bytes, K, E, S, C, sorted, post_padded, ids, x_scale, (uint8_t*)x_perm,
                       scale_perm, row_of_slot);
    return hipGetLastError();
}

// Gradient of the unpermute-combine (the Megatron section of the same page:
// permute and unpermute are each other's gradients, so the gradient of the
// weighted unpermute is a weighted permute of d_out).  One wave per row r < P:
// the row's slot s = sorted[r] gets
//   d_y_perm[r] = w[s] * d_out[s / K]          (fp32 product; fp32 or bf16 out)
//   d_w[s]      = <d_out[s / K], y_perm[r]>    (fp32: lane partial sums, then
//                                                the wave's butterfly)
// and a padding row gets zeros.  A slot whose id is outside [0,E) is never
// placed: the thread of that slot writes its zero d_w (disjoint from the row
// writers, as for row_of_slot above).
template <bool kBf16>
__global__ void __launch_bounds__(kPermThreads)
unpermute_combine_bwd_kernel(int K, int E, int H, int64_t S, int64_t C, const float* __restrict__ d_out,
                             const float* __restrict__ y_perm, const float* __restrict__ w,
                             const int32_t* __restrict__ ids, const int32_t* __restrict__ sorted,
                             const int32_t* __restrict__ post_padded, void* __restrict__ d_y_perm,
                             float* __restrict__ d_w) {
    const int lane = lane_id();
    const int64_t g = (int64_t)blockIdx.x * kPermThreads + threadIdx.x;
    if (g < S) {
        const int e = ids[g];
        if (e < 0 || e >= E) d_w[g] = 0.f;
    }
    const int64_t r = (int64_t)blockIdx.x * kPermRowsPerWg + threadIdx.x / kWave;
    if (r >= C || r >= post_padded[0]) return;
    const int slot = sorted[r];
    const bool placed = slot >= 0 && slot < S;
    const int nq = H / 4;
    const float wk = placed ? w[slot] : 0.f;
    const f32x4_t* go = (const f32x4_t*)(d_out + (placed ? (int64_t)(slot / K) * H : 0));
    const f32x4_t* yr = (const f32x4_t*)(y_perm + r * H);
    float dot = 0.f;
    for (int c = lane; c < nq; c += kWave) {
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
        if (placed) {
            const f32x4_t gv = go[c];
            const f32x4_t yv = __builtin_nontemporal_load(yr + c);
            dot += (gv[0] * yv[0] + gv[1] * yv[1]) + (gv[2] * yv[2] + gv[3] * yv[3]);
            o = f32x4_t{wk * gv[0], wk * gv[1], wk * gv[2], wk * gv[3]};
        }
        if (kBf16) {
            const uint32_t lo = (uint32_t)f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16);
            *(uint2*)((uint16_t*)d_y_perm + r * H + 4 * c) = make_uint2(lo, hi);
        } else {
            *(f32x4_t*)((float*)d_y_perm + r * H + 4 * c) = o;
        }
    }
    if (!placed) return;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
    if (lane == 0) d_w[slot] = dot;
}

hipError_t launch_unpermute_combine_backward(int K, int E, int H, int64_t S, int64_t C, const float* d_out,
                                             const float* y_perm, const float* w, const int32_t* ids,
                                             const int32_t* sorted, const int32_t* post_padded, int out_bf16,
                                             void* d_y_perm, float* d_w, hipStream_t stream) {
    if (C == 0) return hipSuccess;
    const int64_t nwg = (C + kPermRowsPerWg - 1) / kPermRowsPerWg;   // also covers the S slots: C >= S
    if (out_bf16)
        hipLaunchKernelGGL(unpermute_combine_bwd_kernel<true>, dim3((unsigned)nwg), dim3(kPermThreads), 0, stream,
                           K, E, H, S, C, d_out, y_perm, w, ids, sorted, post_padded, d_y_perm, d_w);
    else
        hipLaunchKernelGGL(unpermute_combine_bwd_kernel<false>, dim3((unsigned)nwg), dim3(kPermThreads), 0, stream,
                           K, E, H, S, C, d_out, y_perm, w, ids, sorted, post_padded, d_y_perm, d_w);
    return hipGetLastError();
}

}  // namespace moe
