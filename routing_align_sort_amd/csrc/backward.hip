// Backward of the MoE layer (training) for gfx950: bf16 weights and
// activations, fp32 gradients.
//
// What it computes: the derivative of the forward -- "AMD GPU ... 7x faster
// ... efficient MoE with any number of experts" (dignews.cc), the Megatron
// section (for training, the permute gets its gradient, unpermute) and the
// TransformerEngine paragraph; the X-MoE abstract (taxoreview.com): MoE
// training on AMD GPUs.  The selection is held fixed and the intermediate's
// bf16 rounding is passed straight through:
//   d_w[t,k] = <d_out[t], y_slots[t*K+k]>,  dy = w[t,k] * d_out[t]
//   dW2[e]  += dy^T a~,   d_a = dy W2[e]
//   d_g = d_a * u * SiLU'(g),  d_u = d_a * SiLU(g)
//   dW13[e] += [d_g d_u]^T x,  dx[t] += [d_g d_u] W13[e]
//   routing: d_logits from d_w through softmax or sigmoid (+ renormalisation)
//
// The path: rows are moved into the sorted order (permute), the gate/up
// values are recomputed (NT GEMM per M block), the data gradients are NN
// GEMMs per M block against the weight slabs in their own layout, and the
// weight gradients are NN GEMMs per expert over the expert's contiguous
// segment: transposed dy / [d_g d_u] against the activation rows.
// Every GEMM operand is bf16 (dy and [d_g d_u] rounded once), every
// accumulation fp32.  Needs block_size_m a multiple of 64 (each expert's
// segment is then a whole number of 64-element K-steps).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kBwdThreads = 256;

// ------------------------------------------------------------- transpose --
// dst[b][c][r] = src[b][r][c] for r < rows (from *rows_dev when given),
// c < cols; src pitch cols, dst pitch ldd.  64 x 64 tiles through LDS, 16-byte
// global loads and stores (cols and ldd multiples of 8, rows tile-padded by
// the caller's buffers only up to the real rows).
constexpr int kTp = 64;
__global__ void __launch_bounds__(kBwdThreads)
transpose_bf16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int rows, int cols,
                      int64_t ldd, int64_t src_batch, int64_t dst_batch, int ntc, const int32_t* rows_dev) {
    __shared__ uint16_t tile[kTp][kTp + 2];
    const int nr = rows_dev ? min(rows, rows_dev[0]) : rows;
    const int tr = blockIdx.x / ntc, tc = blockIdx.x % ntc;
    const int r0 = tr * kTp, c0 = tc * kTp;
    if (r0 >= nr) return;
    const uint16_t* s = src + blockIdx.y * src_batch;
    uint16_t* d = dst + blockIdx.y * dst_batch;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 2; ++j) {                          // 64 rows x 8 chunks of 8 elements
        const int r = tid / 8 + 32 * j, cc = (tid % 8) * 8;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r0 + r < nr && c0 + cc < cols) v = *(const uint4*)(s + (int64_t)(r0 + r) * cols + c0 + cc);
        const uint16_t* e = (const uint16_t*)&v;
#pragma unroll
        for (int q = 0; q < 8; ++q) tile[r][cc + q] = e[q];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {                          // 64 columns x 8 chunks of 8 rows
        const int c = tid / 8 + 32 * j, rr = (tid % 8) * 8;
        if (c0 + c >= cols || r0 + rr >= nr) continue;
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = (r0 + rr + q < nr) ? tile[rr + q][c] : (uint16_t)0;
        *(uint4*)(d + (int64_t)(c0 + c) * ldd + r0 + rr) = *(const uint4*)e;
    }
}

static hipError_t transpose(const uint16_t* src, uint16_t* dst, int rows, int cols, int64_t ldd, int batch,
                            int64_t src_batch, int64_t dst_batch, const int32_t* rows_dev, hipStream_t stream) {
    const int ntr = (rows + kTp - 1) / kTp, ntc = (cols + kTp - 1) / kTp;
    if (ntr == 0 || ntc == 0 || batch == 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(ntr * ntc), (unsigned)batch), dim3(kBwdThreads), 0,
                       stream, src, dst, rows, cols, ldd, src_batch, dst_batch, ntc, rows_dev);
    return hipGetLastError();
}

// ------------------------------------------------------- combine backward --
// One workgroup per token: for every slot, d_w = <d_out[t], y_slots[slot]>
// (fp32, summed per thread then across the workgroup) and the slot's dy row
// w * d_out[t] rounded to bf16 (zero for a skipped slot).
__global__ void __launch_bounds__(kBwdThreads)
combine_bwd_kernel(int K, int E, int H, const int32_t* __restrict__ ids, const float* __restrict__ w,
                   const float* __restrict__ y, const float* __restrict__ d_out, float* __restrict__ d_w,
                   uint16_t* __restrict__ dy) {
    __shared__ float red[kBwdThreads / kWave];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float* go = d_out + (int64_t)t * H;
    for (int k = 0; k < K; ++k) {
        const int64_t i = (int64_t)t * K + k;
        const int e = ids[i];
        const bool ok = e >= 0 && e < E;
        const float wk = ok ? w[i] : 0.f;
        float dot = 0.f;
        for (int h = tid * 4; h < H; h += kBwdThreads * 4) {
            const f32x4_t g = *(const f32x4_t*)(go + h);
            if (ok) {
                const f32x4_t v = *(const f32x4_t*)(y + i * H + h);
                dot += g[0] * v[0] + g[1] * v[1] + g[2] * v[2] + g[3] * v[3];
            }
            uint2 o;
            o.x = (uint32_t)f32_to_bf16_bits(wk * g[0]) | ((uint32_t)f32_to_bf16_bits(wk * g[1]) << 16);
            o.y = (uint32_t)f32_to_bf16_bits(wk * g[2]) | ((uint32_t)f32_to_bf16_bits(wk * g[3]) << 16);
            *(uint2*)(dy + i * H + h) = o;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
        if (lane_id() == 0) red[tid / kWave] = dot;
        __syncthreads();
        if (tid == 0) d_w[i] = ok ? (red[0] + red[1]) + (red[2] + red[3]) : 0.f;
        __syncthreads();
    }
}

// -------------------------------------------------------- SwiGLU backward --
// Row r < P of the sorted layout: from the recomputed gate/up values gu
// [C,2I] (fp32) and d_a [C,I]: a~ = bf16(SiLU(g) u) (as the forward rounds
// it), d_g = d_a u SiLU'(g), d_u = d_a SiLU(g), both rounded to bf16.
__global__ void __launch_bounds__(kBwdThreads)
swiglu_bwd_kernel(int I, const int32_t* __restrict__ post_padded, const float* __restrict__ gu,
                  const float* __restrict__ d_a, uint16_t* __restrict__ a_out, uint16_t* __restrict__ dgu) {
    const int64_t r = blockIdx.x;
    if (r >= post_padded[0]) return;
    const float* gr = gu + r * 2 * I;
    for (int j = threadIdx.x; j < I; j += kBwdThreads) {
        const float g = gr[j], u = gr[I + j], da = d_a[r * I + j];
        const float s = 1.0f / (1.0f + __expf(-g));
        const float silu = g / (1.0f + __expf(-g));         // the forward's SiLU
        a_out[r * I + j] = f32_to_bf16_bits(silu * u);
        dgu[r * 2 * I + j] = f32_to_bf16_bits(da * u * (s * (1.0f + g * (1.0f - s))));
        dgu[r * 2 * I + I + j] = f32_to_bf16_bits(da * silu);
    }
}

// --------------------------------------------------------- routing backward --
// One wave per token, scores in double (as the forward computes them):
// dL/ds_e = c (d_w_k / N - [renorm] sum_j d_w_j s_j / N^2) for the chosen
// e = e_k; softmax: d l = s (dL/ds - <dL/ds, s>); sigmoid: d l = dL/ds s (1-s).
constexpr int kRbMaxPerLane = kRouteMaxExperts / kWave;
__global__ void __launch_bounds__(kBwdThreads)
route_bwd_kernel(RouteArgs a, const float* __restrict__ d_w, float* __restrict__ d_logits) {
    const int t = blockIdx.x * (kBwdThreads / kWave) + threadIdx.x / kWave;
    if (t >= a.T) return;
    const int lane = lane_id(), E = a.E, K = a.K;
    const int KO = K + (a.append_shared ? 1 : 0);
    const float* l = a.logits + (int64_t)t * E;
    const int J = (E + kWave - 1) / kWave;
    double s[kRbMaxPerLane];
    if (a.score == 0) {
        double mx = -1e300;
        for (int j = 0; j < J; ++j) {
            const int e = j * kWave + lane;
            if (e < E) mx = fmax(mx, (double)l[e]);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, kWave));
        double z = 0.0;
#pragma unroll
        for (int j = 0; j < kRbMaxPerLane; ++j) {
            const int e = j * kWave + lane;
            s[j] = (j < J && e < E) ? exp((double)l[e] - mx) : 0.0;
            z += s[j];
        }
        z = wave_sum_f64(z);
#pragma unroll
        for (int j = 0; j < kRbMaxPerLane; ++j) s[j] /= z;
    } else {
#pragma unroll
        for (int j = 0; j < kRbMaxPerLane; ++j) {
            const int e = j * kWave + lane;
            s[j] = (j < J && e < E) ? 1.0 / (1.0 + exp(-(double)l[e])) : 0.0;
        }
    }
    // the chosen experts' scores, known to every lane (K <= 64)
    auto score_of = [&](int e) -> double {
        double v = 0.0;
#pragma unroll
        for (int j = 0; j < kRbMaxPerLane; ++j) v = (j * kWave + lane == e) ? s[j] : v;
        return wave_sum_f64(v);                              // exactly one lane holds it
    };
    double N = 1.0, sdw = 0.0;
    if (a.renormalize) N = 0.0;
    for (int k = 0; k < K; ++k) {
        const int e = a.topk_ids[(int64_t)t * KO + k];
        const double se = score_of(e);
        if (a.renormalize) N += se;
        sdw += (double)d_w[(int64_t)t * KO + k] * se;
    }
    double gs[kRbMaxPerLane];
#pragma unroll
    for (int j = 0; j < kRbMaxPerLane; ++j) gs[j] = 0.0;
    for (int k = 0; k < K; ++k) {
        const int e = a.topk_ids[(int64_t)t * KO + k];
        double v = (double)d_w[(int64_t)t * KO + k] / N;
        if (a.renormalize) v -= sdw / (N * N);
        v *= (double)a.routed_scaling;
#pragma unroll
        for (int j = 0; j < kRbMaxPerLane; ++j)
            if (j * kWave + lane == e) gs[j] += v;
    }
    double dot = 0.0;
    if (a.score == 0) {
#pragma unroll
        for (int j = 0; j < kRbMaxPerLane; ++j) dot += gs[j] * s[j];
        dot = wave_sum_f64(dot);
    }
#pragma unroll
    for (int j = 0; j < kRbMaxPerLane; ++j) {
        const int e = j * kWave + lane;
        if (j < J && e < E) {
            const double d = a.score == 0 ? s[j] * (gs[j] - dot) : gs[j] * s[j] * (1.0 - s[j]);
            d_logits[(int64_t)t * E + e] = (float)d;
        }
    }
}

hipError_t launch_route_backward(const RouteArgs& a, const float* d_w, float* d_logits, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int per = kBwdThreads / kWave;
    hipLaunchKernelGGL(route_bwd_kernel, dim3((unsigned)((a.T + per - 1) / per)), dim3(kBwdThreads), 0, stream, a,
                       d_w, d_logits);
    return hipGetLastError();
}

// ------------------------------------------------------------------ host --
static inline int64_t al256(int64_t v) { return (v + 255) / 256 * 256; }

struct BwdWs {
    uint16_t *x_perm, *dy_slots, *dy_perm, *a_bf, *dgu, *dyt, *dgut;
    float *gu, *d_a, *dxs;
    int32_t *row_of_slot, *row_of_slot2;
};

static BwdWs bwd_ws(void* ws, int64_t T, int64_t K, int64_t E, int64_t H, int64_t I, int64_t C, int64_t* total) {
    uint8_t* p = static_cast<uint8_t*>(ws);
    const int64_t S = T * K;
    BwdWs w;
    auto take = [&](int64_t bytes) { uint8_t* q = p; p += al256(bytes); return q; };
    w.x_perm = (uint16_t*)take(C * H * 2);
    w.dy_slots = (uint16_t*)take(S * H * 2);
    w.dy_perm = (uint16_t*)take(C * H * 2);
    w.gu = (float*)take(C * 2 * I * 4);
    w.d_a = (float*)take(C * I * 4);
    w.a_bf = (uint16_t*)take(C * I * 2);
    w.dgu = (uint16_t*)take(C * 2 * I * 2);
    w.dxs = (float*)take(C * H * 4);
    w.dyt = (uint16_t*)take(H * C * 2);
    w.dgut = (uint16_t*)take(2 * I * C * 2);
    w.row_of_slot = (int32_t*)take(S * 4);
    w.row_of_slot2 = (int32_t*)take(S * 4);
    if (total) *total = p - static_cast<uint8_t*>(ws);
    return w;
}

int64_t ffn_backward_workspace_bytes(int64_t T, int64_t K, int64_t E, int64_t H, int64_t I, int64_t C) {
    int64_t total = 0;
    bwd_ws(nullptr, T, K, E, H, I, C, &total);
    return total;
}

#define MOE_TRY(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) return e_; } while (0)

hipError_t launch_ffn_backward(const BwdArgs& a, void* ws, hipStream_t st) {
    const int64_t S = a.S, C = a.C, H = a.H, I = a.I, E = a.E;
    BwdWs w = bwd_ws(ws, a.T, a.K, E, H, I, C, nullptr);
    const int64_t nblk = C / a.B;
    // 1. rows into the sorted order; the slots' dy rows and the combine weights' gradient
    MOE_TRY(launch_permute_rows(a.x, H * 2, a.K, (int)E, S, C, a.sorted, a.post_padded, a.ids, nullptr, w.x_perm,
                                nullptr, w.row_of_slot, st));
    if (a.T > 0)
        hipLaunchKernelGGL(combine_bwd_kernel, dim3(a.T), dim3(kBwdThreads), 0, st, a.K, (int)E, (int)H, a.ids, a.w,
                           a.y_slots, a.d_out, a.d_w, w.dy_slots);
    MOE_TRY(hipGetLastError());
    MOE_TRY(launch_permute_rows(w.dy_slots, H * 2, 1, (int)E, S, C, a.sorted, a.post_padded, a.ids, nullptr,
                                w.dy_perm, nullptr, w.row_of_slot2, st));
    // 2. the gate/up values: the training forward's, or recomputed (weights as
    //    stored: K-contiguous rows)
    NtGemmArgs g{};
    g.expert_ids = a.expert_ids; g.post_padded = a.post_padded; g.offsets = a.offsets; g.by_block = 1;
    const float* gu = a.gate_up ? a.gate_up : w.gu;
    if (!a.gate_up) {
        g.a = w.x_perm; g.lda = H; g.b = a.w13; g.ldb = H; g.b_group = 2 * I * H; g.c = w.gu; g.ldc = 2 * I;
        g.M = a.B; g.N = (int)(2 * I); g.K = (int)H;
        MOE_TRY(launch_nt_gemm(g, a.B, nblk, st));
    }
    g.M = a.B;
    // 3. d_a = dy W2[e] (W2[e] is [H][I]: the NN form), SwiGLU backward, dx rows = [d_g d_u] W13[e]
    g.a = w.dy_perm; g.lda = H; g.b = a.w2; g.ldb = I; g.b_group = H * I; g.c = w.d_a; g.ldc = I;
    g.N = (int)I; g.K = (int)H;
    MOE_TRY(launch_nn_gemm(g, a.B, nblk, st));
    if (C > 0)
        hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)C), dim3(kBwdThreads), 0, st, (int)I, a.post_padded,
                           gu, (const float*)w.d_a, w.a_bf, w.dgu);
    MOE_TRY(hipGetLastError());
    g.a = w.dgu; g.lda = 2 * I; g.b = a.w13; g.ldb = H; g.b_group = 2 * I * H; g.c = w.dxs; g.ldc = H;
    g.N = (int)H; g.K = (int)(2 * I);
    MOE_TRY(launch_nn_gemm(g, a.B, nblk, st));
    MOE_TRY(launch_unpermute_combine(a.T, a.K, (int)H, w.dxs, nullptr, w.row_of_slot, 0, a.dx, st));
    // 4. weight gradients per expert: transposed dy / [d_g d_u] (K = the expert's rows,
    //    contiguous) against the rows of a~ / x
    MOE_TRY(transpose(w.dy_perm, w.dyt, (int)C, (int)H, C, 1, 0, 0, a.post_padded, st));
    MOE_TRY(transpose(w.dgu, w.dgut, (int)C, (int)(2 * I), C, 1, 0, 0, a.post_padded, st));
    g.by_block = 0;
    g.c_bf16 = a.dw_bf16;
    g.a = w.dyt; g.lda = C; g.b = w.a_bf; g.ldb = I; g.c = (float*)a.dw2; g.ldc = I; g.c_group = H * I;
    g.M = (int)H; g.N = (int)I;
    MOE_TRY(launch_nn_gemm(g, 128, E, st));
    g.a = w.dgut; g.lda = C; g.b = w.x_perm; g.ldb = H; g.c = (float*)a.dw13; g.ldc = H; g.c_group = 2 * I * H;
    g.M = (int)(2 * I); g.N = (int)H;
    MOE_TRY(launch_nn_gemm(g, 128, E, st));
    return hipSuccess;
}

}  // namespace moe
