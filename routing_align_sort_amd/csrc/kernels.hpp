// Host-side launchers of the MoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ----------------------------------------------------------------- routing --
constexpr int kRouteMaxExperts = 1024;
constexpr int kRouteMaxK = 64;
constexpr int kRouteMaxGroups = 64;

struct RouteArgs {
    int T, E, K, score, n_group, topk_group, renormalize, append_shared;
    float routed_scaling;
    const float* logits;
    const float* bias;
    int32_t* topk_ids;
    float* topk_weights;
};
hipError_t launch_route_topk(const RouteArgs& a, hipStream_t stream);
// Per-token E4M3 quantisation of x into the FFN's workspace (codes, scales),
// with the per-row amax of the intermediate cleared (C rows).
struct QuantArgs {
    const uint16_t* x;         // bf16 [T,H]
    int H;
    uint8_t* xq;               // [T,H]
    float* sx;                 // [T]
    uint32_t* amax;            // [C]
    int64_t C;
};
// Routing and the quantisation of the same T tokens in one launch.
hipError_t launch_route_quant(const RouteArgs& a, const QuantArgs& q, hipStream_t stream);

// ------------------------------------------------------------- align&sort --
constexpr int kAlignMaxExperts = 1024;

struct AlignPlan {
    bool single;               // one workgroup, no workspace
    bool masks;                // stable ranks from per-wave LDS masks (else ballots)
    bool merge;                // each workgroup merges the [G,E] counts (else column scans)
    bool tagged;               // merge of tagged count words, no grid barrier (few workgroups)
    int G;                     // workgroups (1, or a multiple of the 8 XCDs)
    int R;                     // slots per thread (chunk = 1024 * R)
    int64_t chunk;
    int64_t workspace_bytes;   // barrier words + counts (+ totals; tagged: 64-bit counts)
};
AlignPlan align_plan(int64_t S, int E);
hipError_t launch_align_sort(const int32_t* ids, int64_t S, int E, int B, int64_t C, int32_t* sorted,
                             int32_t* expert_ids, int32_t* post_padded, int32_t* offsets,
                             void* workspace, hipStream_t stream);
// The no-allocation Align & Sort's fixed scratch (a static device array of
// this many bytes on every device the library runs on): its device address
// on the current device, looked up once per device.
constexpr int64_t kAlignScratchBytes = (int64_t)1088 << 10;
hipError_t align_scratch_address(void** ptr);

// -------------------------------------------------------------- grouped FFN --
struct FfnArgs {
    int T, K, E, H, I, B;
    int64_t S, C;              // slots, capacity (rows of the sorted layout)
    const void* x;
    const void* w13;
    const void* w13_scale;     // fp32 [E,2I] (E4M3) or E8M0 [E,2I,H/32] (E2M1); else unused
    const void* w2;
    const void* w2_scale;      // fp32 [E,H] (E4M3) or E8M0 [E,H,I/32] (E2M1); else unused
    const int32_t* sorted_ids;
    const int32_t* expert_ids;
    const int32_t* post_padded;
    float* y_slots;            // [S,H] by slot, or [C,H] in the sorted row order
    int y_bf16;                // y_slots holds bf16 rows (rounded to nearest even), rows by slot
    int packed;                // weights in the layout written by launch_prepack
    int rows_sorted;           // x is [C,H] in the sorted row order, y written in that order
    int fused;                 // both GEMMs in one persistent launch
    // Top-1 combine in the down GEMM's epilogue (K == 1, rows by token): when
    // top1_out is set, out[t] = top1_w[t] * y of t's slot is written there
    // (bf16 when top1_bf16, else fp32) instead of y_slots, and tokens whose
    // id is outside [0,E) get zero rows.
    const float* top1_w;
    const int32_t* top1_ids;
    void* top1_out;
    int top1_bf16;
    // Training forward: the gate and up values (fp32, after any scales) of
    // sorted row r are written to save_gu[r*2I + j] and [r*2I + I + j] for
    // rows below num_tokens_post_padded, for the backward; null otherwise.
    float* save_gu;
    // the workspace already holds x's codes and scales and a cleared row
    // amax (launch_route_quant): no quantisation launch
    int x_quantized;
};
// The quantisation targets of an E4M3 / E2M1 FFN's workspace for T token rows.
QuantArgs ffn_quant_args(void* ws, const void* x, int64_t T, int64_t H, int64_t I, int64_t C);
// Largest activation operand (bytes of x, or of the intermediate, as one
// GEMM reads it) of the matrix-core kernels: they address it with 32-bit
// offsets.
constexpr int64_t kFfnMaxOperandBytes = (int64_t)1 << 32;
// Workspace layout per dtype path (bytes, each region 256-byte aligned).
// T here is the number of x rows; fused adds the one-stage control block.
int64_t ffn_workspace_bytes(int w_dtype, int64_t T, int64_t H, int64_t I, int64_t C, int fused);
// ev (nullable) = 5 caller-created events recorded at the stage boundaries:
// before quantisation, before gate/up, after gate/up, before down, after down.
hipError_t launch_ffn_f32(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev);
hipError_t launch_ffn_bf16(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev);
hipError_t launch_ffn_fp8(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev);
hipError_t launch_ffn_fp4(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev);

// Rewrites canonical W13 [E,2I,H] and W2 [E,H,I] (bits per element: 16, 8
// or 4) into the packed layout the MFMA kernels stream (same sizes).
hipError_t launch_prepack(int E, int H, int I, int bits, const void* w13, const void* w2, void* w13p,
                          void* w2p, hipStream_t stream);
// Rewrites canonical E8M0 block scales [E,2I,H/32] and [E,H,I/32] into the
// packed order the E2M1 kernels stream (same sizes).
hipError_t launch_prepack_scales(int E, int H, int I, const void* s13, const void* s2, void* s13p, void* s2p,
                                 hipStream_t stream);

inline hipError_t record_stage(hipEvent_t const* ev, int i, hipStream_t s) {
    return ev ? hipEventRecord(ev[i], s) : hipSuccess;
}

// --------------------------------------------------------------- backward --
// Grouped NT GEMM C[m][n] = sum_k A[m][k] B[n][k] (bf16 in, fp32 out); see
// nt_gemm_kernel for the two groupings.
struct NtGemmArgs {
    const uint16_t* a;
    int64_t lda;
    const uint16_t* b;
    int64_t ldb, b_group;
    float* c;                  // fp32 C, or bf16 C at (uint16_t*)c when c_bf16
    int64_t ldc, c_group;
    int M, N, K;
    const int32_t* expert_ids;
    const int32_t* post_padded;
    const int32_t* offsets;
    int by_block;
    int c_bf16;                // NN form only: C rounded to bf16
};
hipError_t launch_nt_gemm(const NtGemmArgs& g, int BM, int64_t groups, hipStream_t stream);
// The NN form C[m][n] = sum_k A[m][k] B[k][n] (B in [K][N], N a multiple of 128),
// same groupings; B_group / ldb address B's rows.
hipError_t launch_nn_gemm(const NtGemmArgs& g, int BM, int64_t groups, hipStream_t stream);

struct BwdArgs {
    int T, K, E, H, I, B;
    int64_t S, C;
    const uint16_t* x;           // [T,H] bf16
    const uint16_t* w13;         // [E,2I,H] bf16
    const uint16_t* w2;          // [E,H,I] bf16
    const int32_t* ids;          // [T,K]
    const float* w;              // [T,K]
    const int32_t* sorted;       // [C]
    const int32_t* expert_ids;   // [C/B]
    const int32_t* post_padded;  // [1]
    const int32_t* offsets;      // [E+1]
    const float* y_slots;        // [S,H] the forward's
    const float* gate_up;        // [C,2I] the training forward's gate and up values, or null (recomputed)
    const float* d_out;          // [T,H]
    float* dx;                   // [T,H]
    void* dw13;                  // [E,2I,H] fp32, or bf16 when dw_bf16
    void* dw2;                   // [E,H,I]
    int dw_bf16;
    float* d_w;                  // [T,K]
};
int64_t ffn_backward_workspace_bytes(int64_t T, int64_t K, int64_t E, int64_t H, int64_t I, int64_t C);
hipError_t launch_ffn_backward(const BwdArgs& a, void* ws, hipStream_t stream);
hipError_t launch_route_backward(const RouteArgs& a, const float* d_w, float* d_logits, hipStream_t stream);

// ----------------------------------------------------------------- combine --
hipError_t launch_combine(int T, int K, int E, int H, const float* y_slots, const float* w,
                          const int32_t* ids, int out_bf16, void* out, hipStream_t stream);
// The same combine over bf16 slot rows (each widened exactly to fp32).
hipError_t launch_combine_bf16_slots(int T, int K, int E, int H, const uint16_t* y_slots, const float* w,
                                     const int32_t* ids, int out_bf16, void* out, hipStream_t stream);
hipError_t launch_unpermute_combine(int T, int K, int H, const float* y_perm, const float* w,
                                    const int32_t* row_of_slot, int out_bf16, void* out, hipStream_t stream);
// Gradient of the unpermute-combine in the permuted layout: d_y_perm rows
// (fp32 or bf16) and the combine weights' gradient.
hipError_t launch_unpermute_combine_backward(int K, int E, int H, int64_t S, int64_t C, const float* d_out,
                                             const float* y_perm, const float* w, const int32_t* ids,
                                             const int32_t* sorted, const int32_t* post_padded, int out_bf16,
                                             void* d_y_perm, float* d_w, hipStream_t stream);

// ----------------------------------------------------------------- permute --
hipError_t launch_permute_rows(const void* x, int64_t row_bytes, int K, int E, int64_t S, int64_t C,
                               const int32_t* sorted, const int32_t* post_padded, const int32_t* ids,
                               const float* x_scale, void* x_perm, float* scale_perm, int32_t* row_of_slot,
                               hipStream_t stream);

}  // namespace moe
