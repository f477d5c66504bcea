/*
 * moe_mi355x.h -- C ABI of the single-GPU Mixture-of-Experts FFN layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer runs as four calls, in order, on one HIP stream:
 *
 *   moe_route_topk   logits [T,E]            -> topk_ids, topk_weights [T,K(+1)]
 *   moe_align_sort   topk_ids                -> sorted_token_ids, expert_ids,
 *                                               num_tokens_post_padded
 *   moe_grouped_ffn  x, expert weights, the sorted layout -> y_slots [T*K, H]
 *   moe_combine      y_slots, topk weights   -> out [T,H]
 *
 * (with top-1 routing, moe_grouped_ffn_top1 does the last two in one call),
 *
 * or, with the rows moved into the sorted order first (the layout a
 * dispatch to expert-owning GPUs sends):
 *
 *   moe_permute_rows       x, the sorted layout -> x_perm [C,H], row_of_slot
 *   moe_grouped_ffn        (row_layout MOE_ROWS_SORTED) x_perm -> y_perm [C,H]
 *   moe_unpermute_combine  y_perm, row_of_slot, topk weights -> out [T,H]
 *
 * Training adds the gradients: moe_ffn_backward (the layer: dx, dw13, dw2,
 * d_topk_weights; after moe_grouped_ffn_train, which keeps the gate and up
 * values for it), moe_route_backward (d_logits), and for the permuted path
 * moe_unpermute_combine_backward (d_y_perm, d_topk_weights) and
 * moe_unpermute_combine with unit weights (the permute's gradient).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named as device pointers must point to device memory of the
 *   current HIP device; tensors are dense and row-major; int32 and fp32
 *   arrays are 4-byte aligned, bf16 arrays 2-byte aligned; x, the weights and
 *   y_slots must be 16-byte aligned with H and I multiples of the tile widths
 *   stated at moe_grouped_ffn.
 * - The caller allocates and owns every buffer.  The library never allocates,
 *   frees or synchronises, and never reads device memory from the host, so a
 *   sequence of calls can be captured into a HIP graph.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   work is enqueued asynchronously on it.  Calls are thread-safe: the
 *   library's only host-side state is one-time per-device set-up (kernel
 *   attributes, device properties, the address of moe_align_sort_noalloc's
 *   scratch), guarded by std::call_once; its only device-side state is that
 *   scratch (see there).  Buffers passed to calls that overlap in time must
 *   not overlap.
 * - Errors: arguments are validated on the host before anything is enqueued;
 *   an invalid call returns a status != MOE_OK and enqueues nothing.  A launch
 *   that fails returns MOE_ERR_HIP.  Data are never an error: expert ids
 *   outside [0,E) are skipped by every step.
 *
 * Notation: T tokens, K experts per token (including an appended shared
 * expert), E experts (weight slabs, including the shared one), H hidden
 * size, I expert intermediate size, B block_size_m (rows per grouped-GEMM
 * block), S = T*K token slots, slot i = t*K + k.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 10

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null pointer, negative or inconsistent size  */
    MOE_ERR_UNSUPPORTED = 2,   /* valid but not built: block size, dtype, E>1024 */
    MOE_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required   */
    MOE_ERR_HIP = 4,           /* a HIP launch failed (no device, bad pointer)  */
    MOE_ERR_SCRATCH_LIMIT = 5  /* input beyond the no-allocation call's scratch */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_FP4_E2M1 = 3 } moe_dtype_t;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_t;

int32_t moe_abi_version(void);
const char *moe_status_string(int32_t status);

/* ------------------------------------------------------------------------ */
/* Top-k routing                                                             */
/* ------------------------------------------------------------------------ */
/*
 * Defined by "AMD GPU ... 7x faster ... efficient MoE with any number of
 * experts" (dignews.cc), opening paragraphs: the gating function sends each
 * token to the experts with the top-K gating scores, DeepSeek V3/R1 adding a
 * per-expert bias to balance load; and its FasterTransformer section (top-k
 * gating softmax and the biased variant).
 *
 * For each token t (row of logits):
 *   score_e = softmax(logits[t])_e  or  1/(1+exp(-logits[t,e]))   (computed in
 *             double, rounded once to fp32)
 *   key_e   = score_e + bias[e]      (fp32; bias may be NULL = 0)
 *   if n_group > 1: experts form n_group equal consecutive groups; a group's
 *             score is the sum of its two largest keys; only the topk_group
 *             best groups stay eligible (ties: lower group index)
 *   the K eligible experts with the largest keys are chosen (ties: lower id),
 *   written in descending key order;
 *   weight  = unbiased score; divided by the sum over the K chosen when
 *             renormalize != 0; times routed_scaling; rounded to fp32.
 *   append_shared != 0 writes one more column (id E, weight 1.0).
 *
 * logits   device fp32 [T,E]        bias device fp32 [E] or NULL
 * topk_ids device int32 [T,K+append_shared]  (row-major, out)
 * topk_weights device fp32 [T,K+append_shared] (out)
 * Limits: 1 <= E <= 1024, 1 <= K <= topk_group*E/n_group, n_group divides E,
 * n_group <= 64.  T = 0 is a no-op.
 */
typedef struct {
    int32_t T, E, K;
    int32_t score;             /* moe_score_t                                  */
    int32_t n_group;           /* 1 = no group limit                           */
    int32_t topk_group;
    int32_t renormalize;
    float routed_scaling;      /* 1.0f for none                                */
    int32_t append_shared;
} moe_route_params_t;

moe_status_t moe_route_topk(const moe_route_params_t *p, const float *logits, const float *bias,
                            int32_t *topk_ids, float *topk_weights, void *stream);

/* ------------------------------------------------------------------------ */
/* Align & Sort                                                              */
/* ------------------------------------------------------------------------ */
/*
 * Defined by the same dignews.cc page: opening paragraphs (sort token slots
 * by expert id, with each expert's run aligned to whole blocks so that the
 * grouped GEMM takes an expert's tokens block by block) and the section on
 * the three-part algorithm (distributed concurrent counting, cumsum, parallel
 * placement).
 *
 * Result (identical to a stable counting sort):
 *   cnt[e]  = number of slots i with topk_ids[i] == e  (ids outside [0,E) skipped)
 *   off[0] = 0, off[e+1] = off[e] + ceil(cnt[e]/B)*B,  P = off[E]
 *   sorted_token_ids[off[e] + r] = the r-th slot (ascending i) with id e;
 *   padding inside each expert's run and the tail [P, C) hold S = T*K;
 *   expert_ids[j] = e for block j in [off[e]/B, off[e+1]/B), -1 for j >= P/B;
 *   num_tokens_post_padded[0] = P; expert_offsets[0..E] = off (if not NULL).
 * Capacity C = moe_align_sort_capacity(T,K,E,B) = B*floor((S + min(E,S)*(B-1))/B),
 * the largest P any id table can produce.
 *
 * topk_ids device int32 [T*K]; sorted_token_ids device int32 [C] (out);
 * expert_ids device int32 [C/B] (out); num_tokens_post_padded device int32 [1]
 * (out); expert_offsets device int32 [E+1] (out) or NULL; workspace device,
 * at least moe_align_sort_workspace_bytes(T,K,E,B) bytes (0 when S <= 4096:
 * NULL allowed), 256-byte aligned.  Its first 4352 bytes hold the words of a
 * grid-wide barrier: the workspace must be zero-filled before its first use
 * (hipMemset, torch.zeros, ...), and every call that completes leaves the
 * barrier's counters zero again, so one workspace serves any number of calls
 * in stream order (concurrent calls need separate workspaces).  The rest is
 * scratch.  Its first int32 is a status word: nonzero means a barrier wait
 * gave up (the workgroups of the launch could not all run at once, which
 * needs other work occupying the device for a long time); the results of
 * that call are then invalid, and the word stays set until the caller
 * clears it.
 * Limits: 1 <= E <= 1024; 1 <= B <= 1024; S + C < 2^31.
 */
int64_t moe_align_sort_capacity(int32_t T, int32_t K, int32_t E, int32_t B);
int64_t moe_align_sort_workspace_bytes(int32_t T, int32_t K, int32_t E, int32_t B);
moe_status_t moe_align_sort(const int32_t *topk_ids, int32_t T, int32_t K, int32_t E, int32_t B,
                            int32_t *sorted_token_ids, int32_t *expert_ids,
                            int32_t *num_tokens_post_padded, int32_t *expert_offsets,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_align_sort_noalloc: moe_align_sort without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments
 * (minus the workspace), same result bits, same errors, plus
 * MOE_ERR_SCRATCH_LIMIT when moe_align_sort_workspace_bytes(T,K,E,B) exceeds
 * moe_align_sort_noalloc_scratch_bytes() (1088 KiB: for example up to 35M
 * slots over 256 experts, or 4.3M over 1024).
 * Its scratch is a fixed device array inside the library; each device the
 * library runs on holds one copy until the process ends, and the call
 * allocates nothing.  Every call on a device uses that device's copy: calls
 * that overlap in time on one device (on different streams, or from
 * different host threads onto one device without ordering) race on it and
 * give wrong results; calls ordered on one stream are safe.
 * The barrier status word of moe_align_sort lives in that array, where the
 * caller cannot read it: a call whose barrier wait gives up returns MOE_OK
 * with invalid results.  The barrier's counters still end at zero (every
 * workgroup arrives at every phase whether or not its wait gave up), so the
 * calls after it are unaffected.
 */
int64_t moe_align_sort_noalloc_scratch_bytes(void);
moe_status_t moe_align_sort_noalloc(const int32_t *topk_ids, int32_t T, int32_t K, int32_t E, int32_t B,
                                    int32_t *sorted_token_ids, int32_t *expert_ids,
                                    int32_t *num_tokens_post_padded, int32_t *expert_offsets,
                                    void *stream);

/* ------------------------------------------------------------------------ */
/* Grouped expert FFN                                                        */
/* ------------------------------------------------------------------------ */
/*
 * Defined by "[Feature]: Add more configuration options for MoE assembly
 * kernels" (ROCm/aiter issue 1248), "Suggestion Description" (gate and up
 * projections with SiLU, the a8w8 mode with per-token fp8 activations, fp8
 * weights and bf16 output, block_size_m rows per block) and the GC-MoE
 * abstract (zhuanzhiai.com: fused SwiGLU, requantisation of the intermediate
 * for the second fp8 GEMM, shared experts).
 *
 * For each block j < P/B with e = expert_ids[j] and each of its rows with
 * slot r = sorted_token_ids[j*B + m] < S, token t = r / K:
 *   a  = SiLU(x[t] . W13[e, 0:I]^T) * (x[t] . W13[e, I:2I]^T)     [I]
 *   y_slots[r] = a . W2[e]^T                                       [H], fp32
 * Rows holding the sentinel and blocks j >= P/B are skipped; rows of y_slots
 * whose slot is never placed are not written.  With p->y_dtype = MOE_BF16
 * the fp32 row is stored rounded to nearest even bf16 (half the bytes the
 * down GEMM writes and the combine reads; moe_combine_slots reads them).
 *   w_dtype = x_dtype = MOE_F32 : fp32 throughout (a kept in fp32)
 *   w_dtype = x_dtype = MOE_BF16: bf16 inputs, fp32 accumulation, a rounded
 *                                 to bf16 between the two GEMMs
 *   w_dtype = MOE_FP8_E4M3, x_dtype = MOE_BF16 (a8w8): x is quantised per
 *     token to OCP E4M3 inside the call (scale = amax/448, code = RNE of
 *     x*(448/amax), saturating); weights are E4M3 codes with one fp32 scale
 *     per output row (w13_scale [E,2I], w2_scale [E,H]); products accumulate
 *     in fp32 and are scaled by the two scales; a is requantised per row the
 *     same way before the down projection.
 *   w_dtype = MOE_FP4_E2M1, x_dtype = MOE_BF16 (a8w4, OCP microscaling FP4
 *     weights; the GC-MoE abstract names FP4 expert weights with block-scaled
 *     products): activations and a are quantised exactly as in a8w8; weights
 *     are E2M1 codes, two per byte with the even column in the low nibble
 *     (w13 [E,2I,H/2] and w2 [E,H,I/2] bytes), and every 32 consecutive
 *     elements of a row share one E8M0 scale byte 2^(s-127) (w13_scale
 *     [E,2I,H/32], w2_scale [E,H,I/32] bytes); products accumulate in fp32
 *     and are scaled by the token's (or a's row's) scale only.
 * x device [T,H] (fp32 or bf16); w13 device [E,2I,H]; w2 device [E,H,I];
 * sorted_token_ids / expert_ids / num_tokens_post_padded as produced by
 * moe_align_sort with the same T,K,E,B; y_slots device [T*K,H] (out) in
 * p->y_dtype: MOE_F32 (0), or MOE_BF16 (bf16, fp8 and MXFP4 weights with
 * MOE_ROWS_BY_TOKEN only; moe_grouped_ffn_train and moe_ffn_backward need
 * MOE_F32, moe_grouped_ffn_top1 writes no y_slots and ignores it; anything
 * else is MOE_ERR_UNSUPPORTED);
 * workspace device, at least moe_grouped_ffn_workspace_bytes(p), 256-byte
 * aligned, clobbered.
 * weight_layout MOE_LAYOUT_PACKED means w13 and w2 were rewritten by
 * moe_prepack_weights (below); fp32 scales of E4M3 weights stay canonical,
 * E8M0 block scales of E2M1 weights must then be rewritten by
 * moe_prepack_block_scales.
 * Limits: B in {16,32,64,128,256}; H a multiple of 256 and I a multiple of 128
 * (fp32: multiples of 64, canonical layout only); E <= 1024; except for fp32,
 * T*H and C*I (C = moe_align_sort_capacity) times the activation element size
 * (2 for bf16, 1 for the quantised paths) at most 4 GiB.  Beyond any limit:
 * MOE_ERR_UNSUPPORTED.
 */
typedef enum { MOE_LAYOUT_CANONICAL = 0, MOE_LAYOUT_PACKED = 1 } moe_weight_layout_t;
/*
 * row_layout MOE_ROWS_BY_TOKEN: x is [T,H] and is gathered through
 * sorted_token_ids; y_slots is [T*K,H] by slot.  MOE_ROWS_SORTED (the
 * receiving side of an expert-parallel dispatch): x is [C,H] already in the
 * sorted order (as moe_permute_rows writes it: row r holds the token of slot
 * sorted_token_ids[r]; rows from num_tokens_post_padded on are never read)
 * and y_slots is [C,H] in the same order, row r written only where
 * sorted_token_ids[r] < T*K.  Not for fp32.
 */
typedef enum { MOE_ROWS_BY_TOKEN = 0, MOE_ROWS_SORTED = 1 } moe_row_layout_t;
/*
 * schedule MOE_SCHEDULE_TWO_LAUNCH: the gate/up GEMM, (E4M3 paths) the
 * intermediate's requantisation and the down GEMM run as separate launches.
 * MOE_SCHEDULE_FUSED (the one-stage form; the aiter issue's Estimated
 * Performance Scaling assumptions note that a fused MoE may keep the
 * intermediate out of global memory, and the dignews.cc page's CK section
 * fuses the MoE's steps into one device pipeline): one persistent launch in
 * which a block's down tiles start as soon as its gate/up tiles are done, and
 * the last of those requantises the block.
 * Both give the same bits.  The fused launch waits on other workgroups
 * with a bounded poll; if a poll gives up (other work holding the device for
 * about a second) it sets a status word in the workspace, at byte offset
 * moe_grouped_ffn_workspace_bytes(p with schedule = MOE_SCHEDULE_TWO_LAUNCH)
 * + 32, and the result is not valid.  Not for fp32.
 */
typedef enum { MOE_SCHEDULE_TWO_LAUNCH = 0, MOE_SCHEDULE_FUSED = 1 } moe_schedule_t;

typedef struct {
    int32_t T, K, E, H, I, B;
    int32_t w_dtype;           /* moe_dtype_t */
    int32_t x_dtype;           /* moe_dtype_t */
    int32_t weight_layout;     /* moe_weight_layout_t of w13 and w2 */
    int32_t row_layout;        /* moe_row_layout_t of x and y_slots */
    int32_t schedule;          /* moe_schedule_t */
    int32_t grad_dtype;        /* moe_dtype_t of moe_ffn_backward's dw13 and dw2: MOE_F32 (0) or MOE_BF16 */
    int32_t y_dtype;           /* moe_dtype_t of y_slots: MOE_F32 (0) or MOE_BF16 */
    int32_t x_quantized;       /* 1: the workspace already holds x's E4M3 codes and
                                  scales, written by moe_route_topk_quantize with
                                  these same parameters; 0: quantised here */
} moe_ffn_params_t;

int64_t moe_grouped_ffn_workspace_bytes(const moe_ffn_params_t *p);
moe_status_t moe_grouped_ffn(const moe_ffn_params_t *p, const void *x, const void *w13,
                             const void *w13_scale, const void *w2, const void *w2_scale,
                             const int32_t *sorted_token_ids, const int32_t *expert_ids,
                             const int32_t *num_tokens_post_padded, void *y_slots,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_route_topk and the per-token activation quantisation of moe_grouped_ffn
 * (E4M3 and E2M1 weights) in one launch.  The two steps are independent: the
 * routing reads the logits, the quantisation reads x.  Launched together they
 * run side by side, and the FFN call then starts with its gate/up GEMM.  The
 * quantisation is the one moe_grouped_ffn runs: per token,
 *   s[t] = max_h |x[t,h]| / 448 (1 when the row is zero),
 *   code = E4M3 nearest-even of x[t,h] * (448 / max_h |x[t,h]|), saturated,
 * the a8w8 per-token activation mode of the aiter issue ("[Feature]: Add more
 * configuration options for MoE assembly kernels", "Suggestion Description").
 * rp, logits, bias, topk_ids, topk_weights as for moe_route_topk.  fp, x,
 * workspace as for the moe_grouped_ffn (or moe_grouped_ffn_top1) call that
 * follows, which must pass the same fp with fp->x_quantized = 1 and the same
 * workspace, and must run after this call (same stream, or ordered by the
 * caller).  Requires fp->w_dtype MOE_FP8_E4M3 or MOE_FP4_E2M1, fp->x_dtype
 * MOE_BF16, MOE_ROWS_BY_TOKEN and fp->T == rp->T (else MOE_ERR_INVALID_ARG);
 * workspace at least moe_grouped_ffn_workspace_bytes(fp) (else
 * MOE_ERR_WORKSPACE).  The codes, scales and the FFN's cleared row-amax
 * buffer go to the workspace; nothing else is written there.  T = 0 is a
 * no-op.
 */
moe_status_t moe_route_topk_quantize(const moe_route_params_t *rp, const float *logits, const float *bias,
                                     int32_t *topk_ids, float *topk_weights, const moe_ffn_params_t *fp,
                                     const void *x, void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_grouped_ffn followed by moe_combine for top-1 routing, in one call.  The
 * combine is defined as for moe_combine (the dignews.cc page, opening
 * paragraphs: a token's output is the gate-weighted result of its chosen
 * experts).  With K == 1 every token has at most one slot, so the sum has one
 * term, and the down GEMM writes it straight into out.
 *   out[t,h] = 0 + topk_weights[t] * y[t,h]   (fp32; the bits of moe_combine)
 *   out[t]   = 0 where topk_ids[t] is outside [0,E)
 * p as for moe_grouped_ffn with p->K == 1 (no appended shared expert),
 * MOE_ROWS_BY_TOKEN and MOE_SCHEDULE_TWO_LAUNCH; bf16, E4M3 or E2M1 weights
 * (fp32: MOE_ERR_UNSUPPORTED).  K != 1 is MOE_ERR_INVALID_ARG.  topk_ids
 * int32 [T] and topk_weights fp32 [T] as moe_route_topk wrote them; out
 * device [T,H] in out_dtype (MOE_F32 or MOE_BF16, bf16 rounded to nearest
 * even).  workspace: moe_grouped_ffn_workspace_bytes(p) bytes.  No y_slots
 * buffer is written.
 */
moe_status_t moe_grouped_ffn_top1(const moe_ffn_params_t *p, const void *x, const void *w13,
                                  const void *w13_scale, const void *w2, const void *w2_scale,
                                  const int32_t *sorted_token_ids, const int32_t *expert_ids,
                                  const int32_t *num_tokens_post_padded, const int32_t *topk_ids,
                                  const float *topk_weights, int32_t out_dtype, void *out,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * One-time weight preparation, off the per-token path: rewrites canonical
 * w13 [E,2I,H] and w2 [E,H,I] (bf16, E4M3 or packed E2M1 pairs, per p->w_dtype;
 * uses p->E, H, I)
 * into the packed layout (same byte sizes) that moe_grouped_ffn streams with
 * one contiguous 1 KB read per load instruction.  The packed layout is a
 * permutation of the bytes, private to this library: produce it only with
 * this call.  Outputs must not alias the inputs.  MOE_ERR_UNSUPPORTED for fp32.
 */
moe_status_t moe_prepack_weights(const moe_ffn_params_t *p, const void *w13, const void *w2,
                                 void *w13_packed, void *w2_packed, void *stream);

/*
 * The companion of moe_prepack_weights for E2M1 weights (p->w_dtype ==
 * MOE_FP4_E2M1, else MOE_ERR_UNSUPPORTED): rewrites the E8M0 block scales
 * w13_scale [E,2I,H/32] and w2_scale [E,H,I/32] (device bytes) into the
 * packed order that moe_grouped_ffn reads beside packed weights (same byte
 * sizes, private to this library).  Outputs must not alias the inputs.
 */
moe_status_t moe_prepack_block_scales(const moe_ffn_params_t *p, const void *w13_scale,
                                      const void *w2_scale, void *w13_scale_packed,
                                      void *w2_scale_packed, void *stream);

/*
 * Profiling form of moe_grouped_ffn: the same work and results, plus five
 * caller-created hipEvent_t handles (events[0..4], passed as void*) recorded on
 * the stream at the stage boundaries -- [0] before the per-token activation
 * quantisation, [1] before the gate/up GEMM, [2] after it, [3] before the down
 * GEMM (after the intermediate's requantisation), [4] after the down GEMM.
 * Stages a dtype path does not have take no time.  For callers that time the
 * stages; the events are only recorded, never created or destroyed here.
 * A NULL array or handle is MOE_ERR_INVALID_ARG.
 */
moe_status_t moe_grouped_ffn_profiled(const moe_ffn_params_t *p, const void *x, const void *w13,
                                      const void *w13_scale, const void *w2, const void *w2_scale,
                                      const int32_t *sorted_token_ids, const int32_t *expert_ids,
                                      const int32_t *num_tokens_post_padded, void *y_slots,
                                      void *workspace, size_t workspace_bytes, void *stream,
                                      void *const *events);

/* ------------------------------------------------------------------------ */
/* Top-k weighted combine                                                    */
/* ------------------------------------------------------------------------ */
/*
 * Defined by the dignews.cc page, opening paragraphs (a token's output is the
 * gate-weighted result of its chosen experts) and the GC-MoE abstract (the
 * shared expert joins the sum; here it is the appended column of weight 1).
 *   out[t,h] = sum over k = 0..K-1 in ascending order, skipping ids outside
 *              [0,E), of topk_weights[t,k] * y_slots[t*K+k, h]   (fp32)
 * y_slots device fp32 [T*K,H]; topk_weights device fp32 [T,K]; topk_ids
 * device int32 [T,K]; out device [T,H] in out_dtype (MOE_F32 or MOE_BF16,
 * bf16 rounded to nearest even).  Limits: H a multiple of 4.
 */
moe_status_t moe_combine(int32_t T, int32_t K, int32_t E, int32_t H, const float *y_slots,
                         const float *topk_weights, const int32_t *topk_ids, int32_t out_dtype,
                         void *out, void *stream);
/*
 * moe_combine_slots: moe_combine with the slot rows in y_dtype.  MOE_F32 is
 * moe_combine itself; MOE_BF16 reads the bf16 rows that moe_grouped_ffn
 * writes with p->y_dtype = MOE_BF16, each value widened exactly to fp32
 * before the same ascending-k fp32 sum.  Limits: H a multiple of 4 (MOE_F32)
 * or of 8 (MOE_BF16); other y_dtype values are MOE_ERR_UNSUPPORTED.
 */
moe_status_t moe_combine_slots(int32_t T, int32_t K, int32_t E, int32_t H, const void *y_slots,
                               int32_t y_dtype, const float *topk_weights, const int32_t *topk_ids,
                               int32_t out_dtype, void *out, void *stream);

/* ------------------------------------------------------------------------ */
/* Permute / unpermute (the dispatch-side data movement)                     */
/* ------------------------------------------------------------------------ */
/*
 * Defined by the dignews.cc page, opening paragraphs: the TransformerEngine
 * paragraph and its "MoE Permute example" figure (a permute moves the rows
 * into expert order and records where each source row went; unpermute is the
 * reverse), and the GC-MoE abstract (expert parallelism pays a token
 * dispatch, the grouped GEMMs and a combine).  The destination order is
 * moe_align_sort's padded layout, so each expert's rows -- and each
 * destination GPU's range of experts -- are contiguous.
 *
 * moe_permute_rows, for r < P = *num_tokens_post_padded (read on the device):
 *   x_perm[r] = x[sorted_token_ids[r] / K] if sorted_token_ids[r] < T*K,
 *               else a zero row;
 *   x_perm_scale[r] = x_scale[that token] or 0 (both NULL to skip);
 * rows from P to C = moe_align_sort_capacity(T,K,E,B) are not written; and
 *   row_of_slot[i] = r with sorted_token_ids[r] = i, or -1 when topk_ids[i]
 *   is outside [0,E) (i < T*K).
 * x device [T, row_bytes] (any element type, row_bytes > 0 and a multiple of
 * 16); topk_ids, sorted_token_ids and num_tokens_post_padded as given to /
 * produced by moe_align_sort with the same T,K,E,B; x_perm device
 * [C, row_bytes]; x_scale device fp32 [T]; x_perm_scale device fp32 [C];
 * row_of_slot device int32 [T*K].
 *
 * moe_unpermute_combine: out[t,h] = sum over k = 0..K-1 in ascending order,
 * skipping row_of_slot[t*K+k] < 0, of topk_weights[t,k] * y_perm[row, h] in
 * fp32 -- the same arithmetic as moe_combine, so on y_perm[r] =
 * y_slots[sorted_token_ids[r]] both give the same bits.  y_perm device fp32
 * [C,H]; out device [T,H] in out_dtype (MOE_F32 or MOE_BF16).  topk_weights
 * NULL means every weight is 1: the sum of a token's rows, which is the
 * gradient of moe_permute_rows (d_x from d_x_perm).  Limits: H a multiple
 * of 4.
 *
 * moe_unpermute_combine_backward: the gradient of moe_unpermute_combine for
 * an upstream d_out [T,H] (the Megatron section of the same page: permute
 * and unpermute are each other's gradients).  For r < P:
 *   d_y_perm[r] = topk_weights[s] * d_out[s / K]   with s = sorted_token_ids[r]
 *                 < T*K (the product in fp32, delivered in d_y_perm_dtype,
 *                 MOE_F32 or MOE_BF16 rounded to nearest even); a zero row
 *                 for a padding row;
 *   d_topk_weights[s] = <d_out[s / K], y_perm[r]>  (fp32 sums);
 * d_topk_weights[i] = 0 for a slot whose topk_ids[i] is outside [0,E); rows
 * from P to C are not written.  d_out device fp32 [T,H]; y_perm device fp32
 * [C,H] (the forward's); topk_weights device fp32 [T,K]; topk_ids,
 * sorted_token_ids, num_tokens_post_padded as for moe_permute_rows with the
 * same T,K,E,B; d_y_perm device [C,H]; d_topk_weights device fp32 [T,K].
 * Limits: H a multiple of 4.
 */
moe_status_t moe_permute_rows(const void *x, int32_t T, int32_t K, int32_t E, int32_t B,
                              int64_t row_bytes, const int32_t *topk_ids,
                              const int32_t *sorted_token_ids, const int32_t *num_tokens_post_padded,
                              const float *x_scale, void *x_perm, float *x_perm_scale,
                              int32_t *row_of_slot, void *stream);
moe_status_t moe_unpermute_combine(int32_t T, int32_t K, int32_t H, const float *y_perm,
                                   const float *topk_weights, const int32_t *row_of_slot,
                                   int32_t out_dtype, void *out, void *stream);
moe_status_t moe_unpermute_combine_backward(int32_t T, int32_t K, int32_t E, int32_t B, int32_t H,
                                            const float *d_out, const float *y_perm,
                                            const float *topk_weights, const int32_t *topk_ids,
                                            const int32_t *sorted_token_ids,
                                            const int32_t *num_tokens_post_padded,
                                            int32_t d_y_perm_dtype, void *d_y_perm,
                                            float *d_topk_weights, void *stream);

/* ------------------------------------------------------------------------ */
/* Backward (training)                                                       */
/* ------------------------------------------------------------------------ */
/*
 * Defined by the dignews.cc page's Megatron section (for training, the
 * permute gets its gradient operation, unpermute) and TransformerEngine
 * paragraph, and the X-MoE abstract (MoE training on AMD GPUs).  The pages
 * give no formulas: these are the exact derivatives of the forward above,
 * with the top-k selection held fixed and the intermediate's rounding passed
 * straight through.
 *
 * moe_ffn_backward, for the upstream gradient d_out of moe_combine's output:
 *   d_topk_weights[t,k] = <d_out[t], y_slots[t*K+k]>     (0 for skipped slots)
 *   dy = topk_weights[t,k] * d_out[t],  a~ = the bf16 intermediate
 *   dw2[e]  = sum over e's slots of dy^T a~
 *   d_a = dy w2[e],  d_g = d_a u SiLU'(g),  d_u = d_a SiLU(g)
 *   dw13[e] = sum over e's slots of [d_g d_u]^T x
 *   dx[t]   = sum over t's slots of [d_g d_u] w13[e]
 * p as for moe_grouped_ffn with bf16 weights and activations, canonical
 * weight layout, MOE_ROWS_BY_TOKEN, MOE_SCHEDULE_TWO_LAUNCH; B in
 * {64,128,256}; H and I multiples of 256.  x, w13, w2, topk_ids,
 * topk_weights: the forward's inputs; sorted_token_ids, expert_ids,
 * num_tokens_post_padded and expert_offsets [E+1]: moe_align_sort's outputs
 * (expert_offsets required here); y_slots: the forward's moe_grouped_ffn
 * output; gate_up: the training forward's gate and up values
 * (moe_grouped_ffn_train), or NULL to recompute them from x and w13 (the
 * same products, the backward's own GEMM); d_out device fp32 [T,H].
 * Outputs (device, overwritten): dx fp32 [T,H]; dw13 [E,2I,H] and dw2
 * [E,H,I] in p->grad_dtype (MOE_F32, or MOE_BF16: the fp32 sums rounded once
 * to nearest even, half the bytes to write; other types MOE_ERR_UNSUPPORTED);
 * d_topk_weights fp32 [T,K].  GEMM operands are bf16 (dy and [d_g d_u]
 * rounded once), accumulation fp32.  workspace: at
 * least moe_ffn_backward_workspace_bytes(p) bytes, 256-byte aligned.
 *
 * moe_grouped_ffn_train: moe_grouped_ffn (bf16 weights and activations,
 * MOE_ROWS_BY_TOKEN, MOE_SCHEDULE_TWO_LAUNCH; else MOE_ERR_UNSUPPORTED) that
 * also writes what the backward reads of the forward: for every sorted row r
 * below num_tokens_post_padded, gate_up[r, j] = g and gate_up[r, I + j] = u,
 * the fp32 products x·w13[e] before the SwiGLU (gate_up device fp32 [C,2I],
 * C = moe_align_sort_capacity; rows from P on are not written).  y_slots as
 * for moe_grouped_ffn; workspace moe_grouped_ffn_workspace_bytes(p).
 *
 * moe_route_backward: d_logits [T,E] (device fp32) for d_topk_weights over
 * the routed columns (an appended shared column has no gradient):
 *   s = softmax(logits) or sigmoid(logits) (double), w_k = c s_{e_k} / N,
 *   N = sum of s over the chosen experts when renormalising, else 1;
 *   dL/ds_e = c (d_w_k / N - [renormalise] sum_j d_w_j s_{e_j} / N^2);
 *   softmax: d_logits = s (dL/ds - <dL/ds, s>); sigmoid: dL/ds s (1 - s).
 * p as given to moe_route_topk; topk_ids [T,K(+1)] its output.
 */
int64_t moe_ffn_backward_workspace_bytes(const moe_ffn_params_t *p);
moe_status_t moe_ffn_backward(const moe_ffn_params_t *p, const void *x, const void *w13, const void *w2,
                              const int32_t *topk_ids, const float *topk_weights,
                              const int32_t *sorted_token_ids, const int32_t *expert_ids,
                              const int32_t *num_tokens_post_padded, const int32_t *expert_offsets,
                              const float *y_slots, const float *gate_up, const float *d_out,
                              float *dx, void *dw13, void *dw2, float *d_topk_weights,
                              void *workspace, size_t workspace_bytes, void *stream);
moe_status_t moe_grouped_ffn_train(const moe_ffn_params_t *p, const void *x, const void *w13,
                                   const void *w2, const int32_t *sorted_token_ids,
                                   const int32_t *expert_ids, const int32_t *num_tokens_post_padded,
                                   float *y_slots, float *gate_up, void *workspace,
                                   size_t workspace_bytes, void *stream);
moe_status_t moe_route_backward(const moe_route_params_t *p, const float *logits,
                                const int32_t *topk_ids, const float *d_topk_weights, float *d_logits,
                                void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
