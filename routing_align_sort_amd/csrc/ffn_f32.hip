// Block-aligned grouped expert FFN in fp32 (the tiny-config path).
//
// Same computation as the bf16 path (the aiter issue's "Suggestion
// Description": gate and up projections, SiLU(gate)*up, down projection, one
// expert per block of block_size_m sorted rows), with fp32 operands and an
// fp32 intermediate.  On MI355X fp32 matrix-core throughput equals the fp32
// vector rate, so this path uses plain FMAs: one thread per output element,
// a workgroup per (block, 64 columns).  It serves small fp32 problems.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kF32Threads = 256;
constexpr int kF32Cols = 64;

__global__ void __launch_bounds__(kF32Threads)
ffn_f32_stage1(FfnArgs a, float* __restrict__ h_out, int nN) {
    const int mb = blockIdx.x / nN, nt = blockIdx.x % nN;
    const int P = a.post_padded[0];
    const int B = a.B;
    if (mb * B >= P) return;
    const int e = a.expert_ids[mb];
    const int H = a.H, I = a.I;
    const int c = nt * kF32Cols + threadIdx.x % kF32Cols;
    const float* wg = (const float*)a.w13 + ((int64_t)e * 2 * I + c) * H;
    const float* wu = wg + (int64_t)I * H;
    for (int m = threadIdx.x / kF32Cols; m < B; m += kF32Threads / kF32Cols) {
        const int slot = a.sorted_ids[(int64_t)mb * B + m];
        float g = 0.f, u = 0.f;
        if (slot < a.S) {
            const float* xr = (const float*)a.x + (int64_t)(slot / a.K) * H;
            for (int h = 0; h < H; ++h) {
                g = fmaf(xr[h], wg[h], g);
                u = fmaf(xr[h], wu[h], u);
            }
        }
        h_out[((int64_t)mb * B + m) * I + c] = g / (1.0f + expf(-g)) * u;
    }
}

__global__ void __launch_bounds__(kF32Threads)
ffn_f32_stage2(FfnArgs a, const float* __restrict__ h_in, int nN) {
    const int mb = blockIdx.x / nN, nt = blockIdx.x % nN;
    const int P = a.post_padded[0];
    const int B = a.B;
    if (mb * B >= P) return;
    const int e = a.expert_ids[mb];
    const int H = a.H, I = a.I;
    const int c = nt * kF32Cols + threadIdx.x % kF32Cols;
    const float* wd = (const float*)a.w2 + ((int64_t)e * H + c) * I;
    for (int m = threadIdx.x / kF32Cols; m < B; m += kF32Threads / kF32Cols) {
        const int slot = a.sorted_ids[(int64_t)mb * B + m];
        if (slot >= a.S) continue;
        const float* hr = h_in + ((int64_t)mb * B + m) * I;
        float y = 0.f;
        for (int j = 0; j < I; ++j) y = fmaf(hr[j], wd[j], y);
        a.y_slots[(int64_t)slot * H + c] = y;
    }
}

hipError_t launch_ffn_f32(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    float* h = static_cast<float*>(ws);                     // [C, I] fp32
    const int nMB = (int)(a.C / a.B);
    const int nN1 = a.I / kF32Cols, nN2 = a.H / kF32Cols;
    hipError_t err;
    if ((err = record_stage(ev, 0, stream)) != hipSuccess) return err;
    if ((err = record_stage(ev, 1, stream)) != hipSuccess) return err;
    if (nMB * nN1 > 0)
        hipLaunchKernelGGL(ffn_f32_stage1, dim3(nMB * nN1), dim3(kF32Threads), 0, stream, a, h, nN1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = record_stage(ev, 2, stream)) != hipSuccess) return err;
    if ((err = record_stage(ev, 3, stream)) != hipSuccess) return err;
    if (nMB * nN2 > 0)
        hipLaunchKernelGGL(ffn_f32_stage2, dim3(nMB * nN2), dim3(kF32Threads), 0, stream, a,
                           (const float*)h, nN2);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return record_stage(ev, 4, stream);
}

}  // namespace moe
