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

}  // namespace moe
