// The C ABI (include/moe_mi355x.h): host-side validation, sizing and launch.
// Nothing here allocates, synchronises or reads device memory.
#include "../../include/moe_mi355x.h"
#include "kernels.hpp"

using namespace moe;

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline moe_status_t from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

int64_t capacity(int64_t S, int64_t E, int64_t B) {
    const int64_t n = S < E ? S : E;
    return B * ((S + n * (B - 1)) / B);
}

bool align_args_ok(int32_t T, int32_t K, int32_t E, int32_t B) {
    if (T < 0 || K < 1 || E < 1 || B < 1) return false;
    const int64_t S = (int64_t)T * K;
    return S + capacity(S, E, B) < ((int64_t)1 << 31);
}

bool ffn_block_ok(int32_t B) { return B == 16 || B == 32 || B == 64 || B == 128 || B == 256; }

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int32_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP launch failed";
        case MOE_ERR_SCRATCH_LIMIT: return "input too large for the fixed scratch of the no-allocation call";
        default: return "unknown status";
    }
}

static moe_status_t route_check(const moe_route_params_t* p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T < 0 || p->E < 1 || p->K < 1 || p->n_group < 1 || p->topk_group < 1 ||
        p->topk_group > p->n_group || p->E % p->n_group != 0 ||
        p->K > p->topk_group * (p->E / p->n_group) || (p->score != MOE_SCORE_SOFTMAX && p->score != MOE_SCORE_SIGMOID))
        return MOE_ERR_INVALID_ARG;
    if (p->E > kRouteMaxExperts || p->K > kRouteMaxK || p->n_group > kRouteMaxGroups) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

static RouteArgs route_args(const moe_route_params_t* p, const float* logits, const float* bias,
                            int32_t* topk_ids, float* topk_weights) {
    RouteArgs a;
    a.T = p->T; a.E = p->E; a.K = p->K; a.score = p->score;
    a.n_group = p->n_group; a.topk_group = p->topk_group;
    a.renormalize = p->renormalize != 0; a.append_shared = p->append_shared != 0;
    a.routed_scaling = p->routed_scaling;
    a.logits = logits; a.bias = bias; a.topk_ids = topk_ids; a.topk_weights = topk_weights;
    return a;
}

moe_status_t moe_route_topk(const moe_route_params_t* p, const float* logits, const float* bias,
                            int32_t* topk_ids, float* topk_weights, void* stream) {
    const moe_status_t st = route_check(p);
    if (st != MOE_OK) return st;
    if (p->T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARG;
    return from_hip(launch_route_topk(route_args(p, logits, bias, topk_ids, topk_weights), as_stream(stream)));
}

int64_t moe_align_sort_capacity(int32_t T, int32_t K, int32_t E, int32_t B) {
    if (!align_args_ok(T, K, E, B)) return -1;
    return capacity((int64_t)T * K, E, B);
}

int64_t moe_align_sort_workspace_bytes(int32_t T, int32_t K, int32_t E, int32_t B) {
    if (!align_args_ok(T, K, E, B)) return -1;
    return align_plan((int64_t)T * K, E).workspace_bytes;
}

moe_status_t moe_align_sort(const int32_t* topk_ids, int32_t T, int32_t K, int32_t E, int32_t B,
                            int32_t* sorted_token_ids, int32_t* expert_ids,
                            int32_t* num_tokens_post_padded, int32_t* expert_offsets,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (!align_args_ok(T, K, E, B)) return MOE_ERR_INVALID_ARG;
    if (E > kAlignMaxExperts || B > 1024) return MOE_ERR_UNSUPPORTED;
    const int64_t S = (int64_t)T * K;
    const int64_t C = capacity(S, E, B);
    if (!num_tokens_post_padded || (S > 0 && !topk_ids) || (C > 0 && (!sorted_token_ids || !expert_ids)))
        return MOE_ERR_INVALID_ARG;
    const int64_t need = align_plan(S, E).workspace_bytes;
    if (need > 0 && (!workspace || (int64_t)workspace_bytes < need)) return MOE_ERR_WORKSPACE;
    return from_hip(launch_align_sort(topk_ids, S, E, B, C, sorted_token_ids, expert_ids,
                                      num_tokens_post_padded, expert_offsets, workspace, as_stream(stream)));
}

int64_t moe_align_sort_noalloc_scratch_bytes(void) { return kAlignScratchBytes; }

moe_status_t moe_align_sort_noalloc(const int32_t* topk_ids, int32_t T, int32_t K, int32_t E, int32_t B,
                                    int32_t* sorted_token_ids, int32_t* expert_ids,
                                    int32_t* num_tokens_post_padded, int32_t* expert_offsets, void* stream) {
    if (!align_args_ok(T, K, E, B)) return MOE_ERR_INVALID_ARG;
    if (E > kAlignMaxExperts || B > 1024) return MOE_ERR_UNSUPPORTED;
    const int64_t S = (int64_t)T * K;
    const int64_t C = capacity(S, E, B);
    if (!num_tokens_post_padded || (S > 0 && !topk_ids) || (C > 0 && (!sorted_token_ids || !expert_ids)))
        return MOE_ERR_INVALID_ARG;
    if (align_plan(S, E).workspace_bytes > kAlignScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
    void* scratch = nullptr;                       // this device's copy of the fixed array
    const hipError_t err = align_scratch_address(&scratch);
    if (err != hipSuccess) return MOE_ERR_HIP;
    return from_hip(launch_align_sort(topk_ids, S, E, B, C, sorted_token_ids, expert_ids,
                                      num_tokens_post_padded, expert_offsets, scratch, as_stream(stream)));
}

static moe_status_t ffn_check(const moe_ffn_params_t* p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T < 0 || p->K < 1 || p->E < 1 || p->H < 1 || p->I < 1 || !align_args_ok(p->T, p->K, p->E, p->B))
        return MOE_ERR_INVALID_ARG;
    const bool f32 = p->w_dtype == MOE_F32 && p->x_dtype == MOE_F32;
    const bool bf16 = p->w_dtype == MOE_BF16 && p->x_dtype == MOE_BF16;
    const bool fp8 = p->w_dtype == MOE_FP8_E4M3 && p->x_dtype == MOE_BF16;
    const bool fp4 = p->w_dtype == MOE_FP4_E2M1 && p->x_dtype == MOE_BF16;
    if (!(f32 || bf16 || fp8 || fp4)) return MOE_ERR_UNSUPPORTED;
    if (!ffn_block_ok(p->B) || p->E > kAlignMaxExperts) return MOE_ERR_UNSUPPORTED;
    if (f32 && (p->H % 64 || p->I % 64)) return MOE_ERR_UNSUPPORTED;
    if (!f32 && (p->H % 256 || p->I % 128)) return MOE_ERR_UNSUPPORTED;
    if (p->weight_layout != MOE_LAYOUT_CANONICAL && p->weight_layout != MOE_LAYOUT_PACKED)
        return MOE_ERR_INVALID_ARG;
    if (f32 && p->weight_layout == MOE_LAYOUT_PACKED) return MOE_ERR_UNSUPPORTED;
    if (p->row_layout != MOE_ROWS_BY_TOKEN && p->row_layout != MOE_ROWS_SORTED) return MOE_ERR_INVALID_ARG;
    if (f32 && p->row_layout == MOE_ROWS_SORTED) return MOE_ERR_UNSUPPORTED;
    if (p->schedule != MOE_SCHEDULE_TWO_LAUNCH && p->schedule != MOE_SCHEDULE_FUSED) return MOE_ERR_INVALID_ARG;
    if (f32 && p->schedule == MOE_SCHEDULE_FUSED) return MOE_ERR_UNSUPPORTED;
    // bf16 slot rows: the matrix-core paths, rows by slot
    if (p->y_dtype != MOE_F32 && p->y_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->y_dtype == MOE_BF16 && (f32 || p->row_layout != MOE_ROWS_BY_TOKEN)) return MOE_ERR_UNSUPPORTED;
    // activations quantised by moe_route_topk_quantize: E4M3 codes of x by token
    if (p->x_quantized != 0 && p->x_quantized != 1) return MOE_ERR_INVALID_ARG;
    if (p->x_quantized && (!(fp8 || fp4) || p->row_layout != MOE_ROWS_BY_TOKEN)) return MOE_ERR_INVALID_ARG;
    if (!f32) {
        // the matrix-core kernels address each GEMM's activation operand
        // (x, then the intermediate) with 32-bit byte offsets
        const int64_t esz = bf16 ? 2 : 1;
        const int64_t C = capacity((int64_t)p->T * p->K, p->E, p->B);
        const int64_t xrows = p->row_layout == MOE_ROWS_SORTED ? C : p->T;
        if (xrows * p->H * esz > kFfnMaxOperandBytes || C * p->I * esz > kFfnMaxOperandBytes)
            return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

// rows of x the FFN reads: tokens, or the sorted layout's capacity
static int64_t ffn_x_rows(const moe_ffn_params_t* p) {
    return p->row_layout == MOE_ROWS_SORTED ? capacity((int64_t)p->T * p->K, p->E, p->B) : p->T;
}

moe_status_t moe_prepack_weights(const moe_ffn_params_t* p, const void* w13, const void* w2,
                                 void* w13_packed, void* w2_packed, void* stream) {
    if (!p || p->E < 1 || p->H < 1 || p->I < 1) return MOE_ERR_INVALID_ARG;
    if (p->w_dtype != MOE_BF16 && p->w_dtype != MOE_FP8_E4M3 && p->w_dtype != MOE_FP4_E2M1)
        return MOE_ERR_UNSUPPORTED;
    if (p->H % 256 || p->I % 128 || p->E > kAlignMaxExperts) return MOE_ERR_UNSUPPORTED;
    if (!w13 || !w2 || !w13_packed || !w2_packed) return MOE_ERR_INVALID_ARG;
    if (w13 == w13_packed || w2 == w2_packed) return MOE_ERR_INVALID_ARG;
    const int bits = p->w_dtype == MOE_BF16 ? 16 : p->w_dtype == MOE_FP8_E4M3 ? 8 : 4;
    return from_hip(launch_prepack(p->E, p->H, p->I, bits, w13, w2, w13_packed, w2_packed, as_stream(stream)));
}

moe_status_t moe_prepack_block_scales(const moe_ffn_params_t* p, const void* w13_scale, const void* w2_scale,
                                      void* w13_scale_packed, void* w2_scale_packed, void* stream) {
    if (!p || p->E < 1 || p->H < 1 || p->I < 1) return MOE_ERR_INVALID_ARG;
    if (p->w_dtype != MOE_FP4_E2M1) return MOE_ERR_UNSUPPORTED;
    if (p->H % 256 || p->I % 128 || p->E > kAlignMaxExperts) return MOE_ERR_UNSUPPORTED;
    if (!w13_scale || !w2_scale || !w13_scale_packed || !w2_scale_packed) return MOE_ERR_INVALID_ARG;
    if (w13_scale == w13_scale_packed || w2_scale == w2_scale_packed) return MOE_ERR_INVALID_ARG;
    return from_hip(launch_prepack_scales(p->E, p->H, p->I, w13_scale, w2_scale, w13_scale_packed,
                                          w2_scale_packed, as_stream(stream)));
}

int64_t moe_grouped_ffn_workspace_bytes(const moe_ffn_params_t* p) {
    if (ffn_check(p) != MOE_OK) return -1;
    const int64_t C = capacity((int64_t)p->T * p->K, p->E, p->B);
    return ffn_workspace_bytes(p->w_dtype, ffn_x_rows(p), p->H, p->I, C, p->schedule == MOE_SCHEDULE_FUSED);
}

// The top-1 combine fused into the down GEMM (moe_grouped_ffn_top1); out
// null for the plain FFN.
struct Top1Out {
    const int32_t* ids;
    const float* w;
    void* out;
    int bf16;
};

static moe_status_t grouped_ffn(const moe_ffn_params_t* p, const void* x, const void* w13,
                                const void* w13_scale, const void* w2, const void* w2_scale,
                                const int32_t* sorted_token_ids, const int32_t* expert_ids,
                                const int32_t* num_tokens_post_padded, void* y_slots, const Top1Out& top1,
                                float* save_gu, void* workspace, size_t workspace_bytes, void* stream,
                                hipEvent_t const* ev) {
    const moe_status_t st = ffn_check(p);
    if (st != MOE_OK) return st;
    const int64_t S = (int64_t)p->T * p->K;
    const int64_t C = capacity(S, p->E, p->B);
    if (S == 0) return MOE_OK;
    if ((!x && !p->x_quantized) || !w13 || !w2 || !sorted_token_ids || !expert_ids || !num_tokens_post_padded ||
        (!y_slots && !top1.out))
        return MOE_ERR_INVALID_ARG;
    if ((p->w_dtype == MOE_FP8_E4M3 || p->w_dtype == MOE_FP4_E2M1) && (!w13_scale || !w2_scale))
        return MOE_ERR_INVALID_ARG;
    const int64_t need =
        ffn_workspace_bytes(p->w_dtype, ffn_x_rows(p), p->H, p->I, C, p->schedule == MOE_SCHEDULE_FUSED);
    if (!workspace || (int64_t)workspace_bytes < need) return MOE_ERR_WORKSPACE;
    FfnArgs a{};
    a.T = p->T; a.K = p->K; a.E = p->E; a.H = p->H; a.I = p->I; a.B = p->B;
    a.S = S; a.C = C;
    a.x = x; a.w13 = w13; a.w13_scale = w13_scale; a.w2 = w2; a.w2_scale = w2_scale;
    a.sorted_ids = sorted_token_ids; a.expert_ids = expert_ids; a.post_padded = num_tokens_post_padded;
    a.y_slots = static_cast<float*>(y_slots);
    a.y_bf16 = p->y_dtype == MOE_BF16 && !top1.out;
    a.packed = p->weight_layout == MOE_LAYOUT_PACKED;
    a.rows_sorted = p->row_layout == MOE_ROWS_SORTED;
    a.fused = p->schedule == MOE_SCHEDULE_FUSED;
    a.top1_w = top1.w; a.top1_ids = top1.ids; a.top1_out = top1.out; a.top1_bf16 = top1.bf16;
    a.save_gu = save_gu;
    a.x_quantized = p->x_quantized;
    hipError_t e;
    if (p->w_dtype == MOE_F32) e = launch_ffn_f32(a, workspace, as_stream(stream), ev);
    else if (p->w_dtype == MOE_BF16) e = launch_ffn_bf16(a, workspace, as_stream(stream), ev);
    else if (p->w_dtype == MOE_FP8_E4M3) e = launch_ffn_fp8(a, workspace, as_stream(stream), ev);
    else e = launch_ffn_fp4(a, workspace, as_stream(stream), ev);
    return from_hip(e);
}

moe_status_t moe_grouped_ffn(const moe_ffn_params_t* p, const void* x, const void* w13,
                             const void* w13_scale, const void* w2, const void* w2_scale,
                             const int32_t* sorted_token_ids, const int32_t* expert_ids,
                             const int32_t* num_tokens_post_padded, void* y_slots, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return grouped_ffn(p, x, w13, w13_scale, w2, w2_scale, sorted_token_ids, expert_ids,
                       num_tokens_post_padded, y_slots, Top1Out{}, nullptr, workspace, workspace_bytes, stream,
                       nullptr);
}

moe_status_t moe_route_topk_quantize(const moe_route_params_t* rp, const float* logits, const float* bias,
                                     int32_t* topk_ids, float* topk_weights, const moe_ffn_params_t* fp,
                                     const void* x, void* workspace, size_t workspace_bytes, void* stream) {
    moe_status_t st = route_check(rp);
    if (st != MOE_OK) return st;
    if ((st = ffn_check(fp)) != MOE_OK) return st;
    if ((fp->w_dtype != MOE_FP8_E4M3 && fp->w_dtype != MOE_FP4_E2M1) || fp->row_layout != MOE_ROWS_BY_TOKEN ||
        fp->T != rp->T)
        return MOE_ERR_INVALID_ARG;
    if (rp->T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights || !x) return MOE_ERR_INVALID_ARG;
    const int64_t C = capacity((int64_t)fp->T * fp->K, fp->E, fp->B);
    const int64_t need = ffn_workspace_bytes(fp->w_dtype, fp->T, fp->H, fp->I, C, fp->schedule == MOE_SCHEDULE_FUSED);
    if (!workspace || (int64_t)workspace_bytes < need) return MOE_ERR_WORKSPACE;
    const QuantArgs q = ffn_quant_args(workspace, x, fp->T, fp->H, fp->I, C);
    return from_hip(
        launch_route_quant(route_args(rp, logits, bias, topk_ids, topk_weights), q, as_stream(stream)));
}

moe_status_t moe_grouped_ffn_train(const moe_ffn_params_t* p, const void* x, const void* w13, const void* w2,
                                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                                   const int32_t* num_tokens_post_padded, float* y_slots, float* gate_up,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    const moe_status_t st = ffn_check(p);
    if (st != MOE_OK) return st;
    if (p->w_dtype != MOE_BF16 || p->x_dtype != MOE_BF16 || p->row_layout != MOE_ROWS_BY_TOKEN ||
        p->schedule != MOE_SCHEDULE_TWO_LAUNCH || p->y_dtype != MOE_F32)
        return MOE_ERR_UNSUPPORTED;
    if ((int64_t)p->T * p->K == 0) return MOE_OK;
    if (!gate_up) return MOE_ERR_INVALID_ARG;
    return grouped_ffn(p, x, w13, nullptr, w2, nullptr, sorted_token_ids, expert_ids, num_tokens_post_padded,
                       y_slots, Top1Out{}, gate_up, workspace, workspace_bytes, stream, nullptr);
}

moe_status_t moe_grouped_ffn_top1(const moe_ffn_params_t* p, const void* x, const void* w13,
                                  const void* w13_scale, const void* w2, const void* w2_scale,
                                  const int32_t* sorted_token_ids, const int32_t* expert_ids,
                                  const int32_t* num_tokens_post_padded, const int32_t* topk_ids,
                                  const float* topk_weights, int32_t out_dtype, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    const moe_status_t st = ffn_check(p);
    if (st != MOE_OK) return st;
    if (p->K != 1) return MOE_ERR_INVALID_ARG;
    if (p->w_dtype == MOE_F32 || p->row_layout != MOE_ROWS_BY_TOKEN || p->schedule != MOE_SCHEDULE_TWO_LAUNCH)
        return MOE_ERR_UNSUPPORTED;
    if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->T == 0) return MOE_OK;
    if (!topk_ids || !topk_weights || !out) return MOE_ERR_INVALID_ARG;
    return grouped_ffn(p, x, w13, w13_scale, w2, w2_scale, sorted_token_ids, expert_ids,
                       num_tokens_post_padded, nullptr, Top1Out{topk_ids, topk_weights, out, out_dtype == MOE_BF16},
                       nullptr, workspace, workspace_bytes, stream, nullptr);
}

moe_status_t moe_grouped_ffn_profiled(const moe_ffn_params_t* p, const void* x, const void* w13,
                                      const void* w13_scale, const void* w2, const void* w2_scale,
                                      const int32_t* sorted_token_ids, const int32_t* expert_ids,
                                      const int32_t* num_tokens_post_padded, void* y_slots,
                                      void* workspace, size_t workspace_bytes, void* stream,
                                      void* const* events) {
    if (!events) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i)
        if (!events[i]) return MOE_ERR_INVALID_ARG;
    return grouped_ffn(p, x, w13, w13_scale, w2, w2_scale, sorted_token_ids, expert_ids,
                       num_tokens_post_padded, y_slots, Top1Out{}, nullptr, workspace, workspace_bytes, stream,
                       reinterpret_cast<hipEvent_t const*>(events));
}

static moe_status_t bwd_check(const moe_ffn_params_t* p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T < 0 || p->K < 1 || p->E < 1 || p->H < 1 || p->I < 1 || !align_args_ok(p->T, p->K, p->E, p->B))
        return MOE_ERR_INVALID_ARG;
    if (p->w_dtype != MOE_BF16 || p->x_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->grad_dtype != MOE_F32 && p->grad_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->y_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;     // the forward's fp32 slot rows are read
    if (p->weight_layout != MOE_LAYOUT_CANONICAL || p->row_layout != MOE_ROWS_BY_TOKEN ||
        p->schedule != MOE_SCHEDULE_TWO_LAUNCH)
        return MOE_ERR_UNSUPPORTED;
    if ((p->B != 64 && p->B != 128 && p->B != 256) || p->E > kAlignMaxExperts) return MOE_ERR_UNSUPPORTED;
    if (p->H % 256 || p->I % 256) return MOE_ERR_UNSUPPORTED;
    const int64_t C = capacity((int64_t)p->T * p->K, p->E, p->B);
    // 32-bit activation offsets inside a GEMM tile: 256 rows of the transposed activations
    if (C * 2 * 256 > kFfnMaxOperandBytes || C * p->H * 2 > kFfnMaxOperandBytes) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int64_t moe_ffn_backward_workspace_bytes(const moe_ffn_params_t* p) {
    if (bwd_check(p) != MOE_OK) return -1;
    const int64_t C = capacity((int64_t)p->T * p->K, p->E, p->B);
    return ffn_backward_workspace_bytes(p->T, p->K, p->E, p->H, p->I, C);
}

moe_status_t moe_ffn_backward(const moe_ffn_params_t* p, const void* x, const void* w13, const void* w2,
                              const int32_t* topk_ids, const float* topk_weights, const int32_t* sorted_token_ids,
                              const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                              const int32_t* expert_offsets, const float* y_slots, const float* gate_up,
                              const float* d_out, float* dx,
                              void* dw13, void* dw2, float* d_topk_weights, void* workspace,
                              size_t workspace_bytes, void* stream) {
    const moe_status_t st = bwd_check(p);
    if (st != MOE_OK) return st;
    if (!x || !w13 || !w2 || !topk_ids || !topk_weights || !sorted_token_ids || !expert_ids ||
        !num_tokens_post_padded || !expert_offsets || !y_slots || !d_out || !dx || !dw13 || !dw2 ||
        !d_topk_weights)
        return MOE_ERR_INVALID_ARG;
    const int64_t S = (int64_t)p->T * p->K;
    const int64_t C = capacity(S, p->E, p->B);
    const int64_t need = ffn_backward_workspace_bytes(p->T, p->K, p->E, p->H, p->I, C);
    if (!workspace || (int64_t)workspace_bytes < need) return MOE_ERR_WORKSPACE;
    BwdArgs a{};
    a.T = p->T; a.K = p->K; a.E = p->E; a.H = p->H; a.I = p->I; a.B = p->B; a.S = S; a.C = C;
    a.x = (const uint16_t*)x; a.w13 = (const uint16_t*)w13; a.w2 = (const uint16_t*)w2;
    a.ids = topk_ids; a.w = topk_weights; a.sorted = sorted_token_ids; a.expert_ids = expert_ids;
    a.post_padded = num_tokens_post_padded; a.offsets = expert_offsets; a.y_slots = y_slots; a.d_out = d_out;
    a.gate_up = gate_up;
    a.dw_bf16 = p->grad_dtype == MOE_BF16;
    a.dx = dx; a.dw13 = dw13; a.dw2 = dw2; a.d_w = d_topk_weights;
    return from_hip(launch_ffn_backward(a, workspace, as_stream(stream)));
}

moe_status_t moe_route_backward(const moe_route_params_t* p, const float* logits, const int32_t* topk_ids,
                                const float* d_topk_weights, float* d_logits, void* stream) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T < 0 || p->E < 1 || p->K < 1 || p->K > p->E || (p->score != MOE_SCORE_SOFTMAX && p->score != MOE_SCORE_SIGMOID))
        return MOE_ERR_INVALID_ARG;
    if (p->E > kRouteMaxExperts || p->K > kRouteMaxK) return MOE_ERR_UNSUPPORTED;
    if (p->T == 0) return MOE_OK;
    if (!logits || !topk_ids || !d_topk_weights || !d_logits) return MOE_ERR_INVALID_ARG;
    RouteArgs a;
    a.T = p->T; a.E = p->E; a.K = p->K; a.score = p->score;
    a.n_group = p->n_group; a.topk_group = p->topk_group;
    a.renormalize = p->renormalize != 0; a.append_shared = p->append_shared != 0;
    a.routed_scaling = p->routed_scaling;
    a.logits = logits; a.bias = nullptr; a.topk_ids = const_cast<int32_t*>(topk_ids); a.topk_weights = nullptr;
    return from_hip(launch_route_backward(a, d_topk_weights, d_logits, as_stream(stream)));
}

moe_status_t moe_permute_rows(const void* x, int32_t T, int32_t K, int32_t E, int32_t B, int64_t row_bytes,
                              const int32_t* topk_ids, const int32_t* sorted_token_ids,
                              const int32_t* num_tokens_post_padded, const float* x_scale, void* x_perm,
                              float* x_perm_scale, int32_t* row_of_slot, void* stream) {
    if (!align_args_ok(T, K, E, B) || row_bytes <= 0 || row_bytes % 16) return MOE_ERR_INVALID_ARG;
    if ((x_scale == nullptr) != (x_perm_scale == nullptr)) return MOE_ERR_INVALID_ARG;
    const int64_t S = (int64_t)T * K;
    if (S == 0) return MOE_OK;
    const int64_t C = capacity(S, E, B);
    if (!x || !topk_ids || !sorted_token_ids || !num_tokens_post_padded || !x_perm || !row_of_slot)
        return MOE_ERR_INVALID_ARG;
    return from_hip(launch_permute_rows(x, row_bytes, K, E, S, C, sorted_token_ids, num_tokens_post_padded,
                                        topk_ids, x_scale, x_perm, x_perm_scale, row_of_slot, as_stream(stream)));
}

moe_status_t moe_unpermute_combine(int32_t T, int32_t K, int32_t H, const float* y_perm,
                                   const float* topk_weights, const int32_t* row_of_slot, int32_t out_dtype,
                                   void* out, void* stream) {
    if (T < 0 || K < 1 || H < 1) return MOE_ERR_INVALID_ARG;
    if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (H % 4) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!y_perm || !row_of_slot || !out) return MOE_ERR_INVALID_ARG;   // topk_weights NULL: weight 1
    return from_hip(launch_unpermute_combine(T, K, H, y_perm, topk_weights, row_of_slot, out_dtype == MOE_BF16,
                                             out, as_stream(stream)));
}

moe_status_t moe_unpermute_combine_backward(int32_t T, int32_t K, int32_t E, int32_t B, int32_t H,
                                            const float* d_out, const float* y_perm, const float* topk_weights,
                                            const int32_t* topk_ids, const int32_t* sorted_token_ids,
                                            const int32_t* num_tokens_post_padded, int32_t d_y_perm_dtype,
                                            void* d_y_perm, float* d_topk_weights, void* stream) {
    if (!align_args_ok(T, K, E, B) || H < 1) return MOE_ERR_INVALID_ARG;
    if (d_y_perm_dtype != MOE_F32 && d_y_perm_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (H % 4) return MOE_ERR_UNSUPPORTED;
    const int64_t S = (int64_t)T * K;
    if (S == 0) return MOE_OK;
    if (!d_out || !y_perm || !topk_weights || !topk_ids || !sorted_token_ids || !num_tokens_post_padded ||
        !d_y_perm || !d_topk_weights)
        return MOE_ERR_INVALID_ARG;
    const int64_t C = capacity(S, E, B);
    return from_hip(launch_unpermute_combine_backward(K, E, H, S, C, d_out, y_perm, topk_weights, topk_ids,
                                                      sorted_token_ids, num_tokens_post_padded,
                                                      d_y_perm_dtype == MOE_BF16, d_y_perm, d_topk_weights,
                                                      as_stream(stream)));
}

moe_status_t moe_combine(int32_t T, int32_t K, int32_t E, int32_t H, const float* y_slots,
                         const float* topk_weights, const int32_t* topk_ids, int32_t out_dtype, void* out,
                         void* stream) {
    if (T < 0 || K < 1 || E < 1 || H < 1) return MOE_ERR_INVALID_ARG;
    if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (H % 4) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!y_slots || !topk_weights || !topk_ids || !out) return MOE_ERR_INVALID_ARG;
    return from_hip(launch_combine(T, K, E, H, y_slots, topk_weights, topk_ids, out_dtype == MOE_BF16, out,
                                   as_stream(stream)));
}

moe_status_t moe_combine_slots(int32_t T, int32_t K, int32_t E, int32_t H, const void* y_slots, int32_t y_dtype,
                               const float* topk_weights, const int32_t* topk_ids, int32_t out_dtype, void* out,
                               void* stream) {
    if (y_dtype == MOE_F32)
        return moe_combine(T, K, E, H, static_cast<const float*>(y_slots), topk_weights, topk_ids, out_dtype, out,
                           stream);
    if (y_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (T < 0 || K < 1 || E < 1 || H < 1) return MOE_ERR_INVALID_ARG;
    if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (H % 8) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!y_slots || !topk_weights || !topk_ids || !out) return MOE_ERR_INVALID_ARG;
    return from_hip(launch_combine_bf16_slots(T, K, E, H, static_cast<const uint16_t*>(y_slots), topk_weights,
                                              topk_ids, out_dtype == MOE_BF16, out, as_stream(stream)));
}

}  // extern "C"
