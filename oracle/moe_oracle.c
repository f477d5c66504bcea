/*
 * moe_oracle.c -- plain, slow CPU oracle for the single-GPU Mixture-of-Experts
 * FFN layer: top-k routing, Align & Sort, the grouped SwiGLU expert FFN and the
 * top-k weighted combine.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only callers.  This file shares no
 * code, header, table or constant generator with the HIP library, and the HIP
 * library never calls it.
 *
 * Sources (web pages; sections named as they appear there):
 *   [DIG]  "AMD GPU ... 7x faster, optimised algorithm open-sourced for the
 *          first time: efficient MoE with any number of experts" (dignews.cc
 *          repost of a Xinzhiyuan article), its opening paragraphs on the MoE
 *          layer and Align & Sort, the FasterTransformer section and the
 *          section on the three-part (count / cumsum / placement) algorithm.
 *   [AIT]  "[Feature]: Add more configuration options for MoE assembly
 *          kernels" (ROCm/aiter issue 1248), "Suggestion Description".
 *   [GCM]  GC-MoE abstract (zhuanzhiai.com): fused SwiGLU, requantization and
 *          optional shared experts inside the grouped GEMM.
 *
 * Arithmetic is double unless stated.  Where a floating-point value decides an
 * integer (which experts are chosen, which fp8 code a value gets) the decision
 * is taken on fp32 values, the precision the GPU kernels decide in; each such
 * fp32 value is the correctly rounded image of a double (or a single fp32
 * operation), so both sides see the same bits.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the oracle's parallel loop uses (reported with its timings). */
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }   /* timing only */

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the upper half of an IEEE binary32 pattern. */
double oracle_bf16_decode(uint16_t b) { return (double)f32_from_bits((uint32_t)b << 16); }

/* Round an fp32 value to the nearest bfloat16, ties to the even pattern.
 * Written as the definition: the two bf16 neighbours of v are the pattern with
 * the low 16 bits dropped (towards zero) and the next pattern away from zero;
 * pick the nearer, and on a tie the one whose last kept bit is 0.  A value
 * past the largest finite bf16 by half an ulp or more rounds to infinity. */
uint16_t oracle_bf16_encode(float v)
{
    uint32_t u = bits_from_f32(v);
    if (isnan(v)) return (uint16_t)((u >> 16) | 0x0040u);      /* quiet NaN */
    if (isinf(v)) return (uint16_t)(u >> 16);
    uint32_t lo_pat = u >> 16;                                  /* towards 0 */
    uint32_t hi_pat = lo_pat + 1u;                              /* away from 0 */
    double a = fabs((double)v);
    double lo = fabs(oracle_bf16_decode((uint16_t)lo_pat));
    /* hi may be the infinity pattern; its "value" for the midpoint test is the
     * next step of the binade, lo + ulp. */
    double ulp = ldexp(1.0, (int)((lo_pat >> 7) & 0xFF) - 127 - 7);
    if (((lo_pat >> 7) & 0xFF) == 0) ulp = ldexp(1.0, -126 - 7);   /* subnormal */
    double hi = lo + ulp;
    double dlo = a - lo, dhi = hi - a;
    if (dlo < dhi) return (uint16_t)lo_pat;
    if (dhi < dlo) return (uint16_t)hi_pat;
    return (uint16_t)((lo_pat & 1u) ? hi_pat : lo_pat);
}

/* OCP 8-bit E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits, no infinities, the all-ones magnitude 0x7F is NaN, largest finite
 * magnitude 1.75 * 2^8 = 448. */
double oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, ex = (c >> 3) & 0xF, m = c & 7;
    double mag;
    if (ex == 0xF && m == 7) return NAN;
    if (ex == 0) mag = ldexp((double)m / 8.0, -6);              /* subnormal */
    else mag = ldexp(1.0 + (double)m / 8.0, ex - 7);
    return s ? -mag : mag;
}

/* Nearest E4M3 value to v, ties to the even code, saturating to +-448 for
 * magnitudes beyond the largest finite value; NaN -> 0x7F.  Written as a
 * search over the 127 non-negative finite codes, which are ordered by value. */
uint8_t oracle_e4m3_encode(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = (bits_from_f32(v) >> 31) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int lo = 0, hi = 0x7E;              /* find neighbours: dec(lo) <= a < dec(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double dlo = a - oracle_e4m3_decode((uint8_t)lo);
    double dhi = oracle_e4m3_decode((uint8_t)hi) - a;
    int code;
    if (dlo < dhi) code = lo;
    else if (dhi < dlo) code = hi;
    else code = (lo & 1) ? hi : lo;
    return (uint8_t)(sign | code);
}

/* Array forms of the codecs, for the test suite. */
/* OCP microscaling FP4, E2M1 element: 1 sign bit, 2 exponent bits (bias 1),
 * 1 mantissa bit, no infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 * E8M0 block scale: the power of two 2^(e-127), e = 255 is NaN.  A block of 32
 * consecutive elements of a row shares one scale.  The GC-MoE abstract
 * (zhuanzhiai.com) names FP4 expert weights. */
double oracle_e2m1_decode(uint8_t nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

double oracle_e8m0_decode(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

void oracle_e2m1_decode_array(const uint8_t *nib, int64_t n, double *out)
{ for (int64_t i = 0; i < n; i++) out[i] = oracle_e2m1_decode(nib[i]); }
void oracle_e8m0_decode_array(const uint8_t *e, int64_t n, double *out)
{ for (int64_t i = 0; i < n; i++) out[i] = oracle_e8m0_decode(e[i]); }

void oracle_bf16_encode_array(const float *v, int64_t n, uint16_t *out)
{ for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_encode(v[i]); }
void oracle_bf16_decode_array(const uint16_t *b, int64_t n, double *out)
{ for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_decode(b[i]); }
void oracle_e4m3_encode_array(const float *v, int64_t n, uint8_t *out)
{ for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(v[i]); }
void oracle_e4m3_decode_array(const uint8_t *c, int64_t n, double *out)
{ for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_decode(c[i]); }

/* ------------------------------------------------------------------------ */
/* Top-k routing                                                             */
/* ------------------------------------------------------------------------ */
/*
 * [DIG] opening paragraphs: an MoE layer's gating function routes each token
 * to the experts with the top-K gating scores; DeepSeek V3/R1 add a per-expert
 * bias to those scores to balance load without an auxiliary loss.  [DIG]
 * FasterTransformer section: "topk gating softmax" and its biased variant.
 *
 * Readings (the pages leave these open):
 *   - score: softmax over the E logits, or the logistic sigmoid of each logit;
 *   - the bias only selects: key_e = score_e + bias_e, but the weight of a
 *     chosen expert is its unbiased score;
 *   - group limit (DeepSeek-V3 style, not on the pages): experts fall into
 *     n_group equal groups, a group's score is the sum of its two largest
 *     keys (its single key when a group has one expert), the topk_group best
 *     groups stay and the keys of every other expert are excluded;
 *   - K largest keys are chosen; equal keys go to the lower expert id; the
 *     output columns are in descending key order (ties: ascending id);
 *   - renormalize divides each chosen weight by their sum; the result is then
 *     multiplied by routed_scaling;
 *   - append_shared adds one column with id E and weight 1 (the always-on
 *     shared expert, stored as expert slab E).
 * Scores are computed in double and rounded once to fp32; keys and group
 * scores are single fp32 additions, so the selection is made on fp32 values.
 */
int oracle_route_topk(int T, int E, int K, int score_mode, int n_group, int topk_group,
                      int renormalize, double routed_scaling, int append_shared,
                      const float *logits, const float *bias,
                      int32_t *topk_ids, float *topk_weights)
{
    if (T < 0 || E < 1 || K < 1 || K > E || n_group < 1 || E % n_group != 0 ||
        topk_group < 1 || topk_group > n_group || K > topk_group * (E / n_group))
        return 1;
    int gsize = E / n_group;
    int KO = K + (append_shared ? 1 : 0);
    double *s = (double *)malloc(sizeof(double) * (size_t)E);
    float *key = (float *)malloc(sizeof(float) * (size_t)E);
    char *allowed = (char *)malloc((size_t)E);
    char *taken = (char *)malloc((size_t)E);
    float *gscore = (float *)malloc(sizeof(float) * (size_t)n_group);
    char *gkeep = (char *)malloc((size_t)n_group);
    int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);

    for (int t = 0; t < T; t++) {
        const float *l = logits + (size_t)t * E;
        /* 1. scores, in double */
        if (score_mode == 0) {
            double mx = -INFINITY, z = 0.0;
            for (int e = 0; e < E; e++) if ((double)l[e] > mx) mx = (double)l[e];
            for (int e = 0; e < E; e++) { s[e] = exp((double)l[e] - mx); z += s[e]; }
            for (int e = 0; e < E; e++) s[e] /= z;
        } else {
            for (int e = 0; e < E; e++) s[e] = 1.0 / (1.0 + exp(-(double)l[e]));
        }
        /* 2. selection keys, fp32 */
        for (int e = 0; e < E; e++) {
            float sc = (float)s[e];
            key[e] = bias ? sc + bias[e] : sc;
            allowed[e] = 1;
            taken[e] = 0;
        }
        /* 3. group limit */
        if (n_group > 1) {
            for (int g = 0; g < n_group; g++) {
                int b1 = -1, b2 = -1;           /* two best experts of the group */
                for (int e = g * gsize; e < (g + 1) * gsize; e++) {
                    if (b1 < 0 || key[e] > key[b1]) { b2 = b1; b1 = e; }
                    else if (b2 < 0 || key[e] > key[b2]) { b2 = e; }
                }
                gscore[g] = (b2 >= 0) ? key[b1] + key[b2] : key[b1];
                gkeep[g] = 0;
            }
            for (int r = 0; r < topk_group; r++) {
                int best = -1;
                for (int g = 0; g < n_group; g++)
                    if (!gkeep[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
                gkeep[best] = 1;
            }
            for (int e = 0; e < E; e++) allowed[e] = gkeep[e / gsize];
        }
        /* 4. top-K: K rounds, each takes the largest remaining key (lower id
         *    on ties), which also yields the descending output order. */
        for (int k = 0; k < K; k++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (allowed[e] && !taken[e] && (best < 0 || key[e] > key[best])) best = e;
            taken[best] = 1;
            chosen[k] = best;
        }
        /* 5. weights from the unbiased scores, in double */
        double sum = 0.0;
        for (int k = 0; k < K; k++) sum += s[chosen[k]];
        for (int k = 0; k < K; k++) {
            double w = s[chosen[k]];
            if (renormalize) w /= sum;
            w *= routed_scaling;
            topk_ids[(size_t)t * KO + k] = chosen[k];
            topk_weights[(size_t)t * KO + k] = (float)w;
        }
        /* 6. shared expert column */
        if (append_shared) {
            topk_ids[(size_t)t * KO + K] = E;
            topk_weights[(size_t)t * KO + K] = 1.0f;
        }
    }
    free(s); free(key); free(allowed); free(taken); free(gscore); free(gkeep); free(chosen);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Align & Sort                                                              */
/* ------------------------------------------------------------------------ */
/*
 * [DIG] opening paragraphs: Align & Sort orders the token slots by expert id,
 * and pads ("aligns") every expert's run to whole blocks so that the grouped
 * GEMM takes an expert's tokens block by block.  The three-part algorithm on
 * the same page (count, cumsum, placement) computes exactly this; the plain
 * definition below is a stable counting sort with per-expert padding.
 *
 * Readings: slot i = t*K + k over the row-major [T,K] id table; ids outside
 * [0,E) are neither counted nor placed; slots of one expert keep ascending i;
 * padding and the unused tail hold the sentinel S = T*K; the unused tail of
 * expert_ids holds -1.
 */
int64_t oracle_align_capacity(int64_t S, int64_t E, int64_t B)
{
    /* the largest possible sum over experts of ceil(cnt_e / B) * B */
    int64_t n = S < E ? S : E;
    return B * ((S + n * (B - 1)) / B);
}

int oracle_align_sort(const int32_t *topk_ids, int T, int K, int E, int B,
                      int32_t *sorted_ids, int32_t *expert_ids,
                      int32_t *num_tokens_post_padded, int32_t *expert_offsets)
{
    if (T < 0 || K < 1 || E < 1 || B < 1) return 1;
    int64_t S = (int64_t)T * K;
    int64_t C = oracle_align_capacity(S, E, B);
    int64_t *cnt = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    int64_t *off = (int64_t *)calloc((size_t)E + 1, sizeof(int64_t));
    int64_t *cursor = (int64_t *)calloc((size_t)E, sizeof(int64_t));
    for (int64_t i = 0; i < S; i++) {
        int32_t e = topk_ids[i];
        if (e >= 0 && e < E) cnt[e]++;
    }
    off[0] = 0;
    for (int e = 0; e < E; e++) off[e + 1] = off[e] + (cnt[e] + B - 1) / B * B;
    for (int64_t j = 0; j < C; j++) sorted_ids[j] = (int32_t)S;
    for (int64_t j = 0; j < C / B; j++) expert_ids[j] = -1;
    for (int e = 0; e < E; e++) cursor[e] = off[e];
    for (int64_t i = 0; i < S; i++) {
        int32_t e = topk_ids[i];
        if (e >= 0 && e < E) sorted_ids[cursor[e]++] = (int32_t)i;
    }
    for (int e = 0; e < E; e++)
        for (int64_t j = off[e] / B; j < off[e + 1] / B; j++) expert_ids[j] = e;
    *num_tokens_post_padded = (int32_t)off[E];
    if (expert_offsets)
        for (int e = 0; e <= E; e++) expert_offsets[e] = (int32_t)off[e];
    free(cnt); free(off); free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token fp8 activation quantisation (a8w8)                              */
/* ------------------------------------------------------------------------ */
/*
 * [AIT] Suggestion Description: the a8w8 kernel takes fp8 activations with a
 * scale per token and fp8 weights.  Reading: scale = amax/448 with amax the
 * largest |x| of the token's row (fp32 division); the code of x is the E4M3
 * rounding of x * (448/amax) (fp32 division, fp32 multiply); an all-zero row
 * has scale 1 and all codes 0.
 */
void oracle_quant_row_e4m3(const float *x, int64_t n, uint8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int64_t h = 0; h < n; h++) { float a = fabsf(x[h]); if (a > amax) amax = a; }
    if (amax == 0.0f) {
        for (int64_t h = 0; h < n; h++) q[h] = 0;
        *scale = 1.0f;
        return;
    }
    float inv = 448.0f / amax;
    for (int64_t h = 0; h < n; h++) q[h] = oracle_e4m3_encode(x[h] * inv);
    *scale = amax / 448.0f;
}

void oracle_quant_tokens_e4m3(const uint16_t *x_bf16, int T, int H, uint8_t *q, float *scales)
{
    float *row = (float *)malloc(sizeof(float) * (size_t)H);
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) row[h] = (float)oracle_bf16_decode(x_bf16[(size_t)t * H + h]);
        oracle_quant_row_e4m3(row, H, q + (size_t)t * H, scales + t);
    }
    free(row);
}

/* ------------------------------------------------------------------------ */
/* Expert FFN per token slot, and the top-k combine                          */
/* ------------------------------------------------------------------------ */
/*
 * [DIG] opening paragraphs: the layer is a set of expert FFNs; each token is
 * processed by the FFNs of its chosen experts.  [AIT] Suggestion Description:
 * the experts have both a gate and an up projection and the activation is
 * SiLU ("g1u1 silu"), then the down projection.  [GCM]: SwiGLU, the
 * requantisation of the intermediate for the second fp8 GEMM, and the shared
 * expert.
 *
 * For slot i = t*K + k with e = ids[i] in [0,E):
 *   g_j = sum_h x[t,h] Wg[e,j,h],  u_j = sum_h x[t,h] Wu[e,j,h]   (j < I)
 *   a_j = SiLU(g_j) * u_j = g_j / (1 + exp(-g_j)) * u_j
 *   a_j is rounded to the intermediate type
 *   y_h = sum_j a_j Wd[e,h,j]                                     (h < H)
 *   y_slots[i,h] = (float) y_h
 * Slots whose id is out of range are left untouched.
 *
 * Layouts: x [T,H]; w13 [E,2I,H] with rows [0,I) the gate and [I,2I) the up
 * projection; w2 [E,H,I].  w_dtype: 0 fp32, 1 bf16 bits, 2 E4M3 codes with
 * one fp32 scale per output row (w13_scale [E,2I], w2_scale [E,H]), 3 MXFP4:
 * E2M1 codes two per byte (w13 [E,2I,H/2], w2 [E,H,I/2] bytes) with one E8M0
 * scale per 32 elements of a row (w13_scale [E,2I,H/32], w2_scale [E,H,I/32]
 * bytes).
 * For w_dtype 2 and 3 the activations are the bf16 x quantised per token
 * (above), and the dot products are formed on the decoded values (exact in
 * double; for MXFP4 each weight already carries its block scale) and then
 * multiplied by the token's scale and, for E4M3 weights, the row's scale.
 * inter: 0 keep double (no rounding, used by the oracle's own checks),
 *        1 round to fp32, 2 round to fp32 then to bf16,
 *        3 round to fp32 then requantise the row to E4M3 with a per-row scale
 *          (same rule as the activation quantisation).
 */
static double e2m1_table[16], e8m0_table[256];

static void mx_tables(void)
{
    for (int i = 0; i < 16; i++) e2m1_table[i] = oracle_e2m1_decode((uint8_t)i);
    for (int i = 0; i < 256; i++) e8m0_table[i] = oracle_e8m0_decode((uint8_t)i);
}

/* Element (row, col) of a weight matrix whose rows have `len` elements.
 * w_dtype 3 (MXFP4): two codes per byte along the row, the even column in the
 * low nibble; the scale of columns [32b, 32b+32) of a row is byte b of that
 * row's scale array (len/32 bytes per row); the value includes it. */
static double load_w(int w_dtype, const void *w, const void *wscale, size_t row, int col, int len)
{
    size_t idx = row * (size_t)len + (size_t)col;
    if (w_dtype == 0) return (double)((const float *)w)[idx];
    if (w_dtype == 1) return oracle_bf16_decode(((const uint16_t *)w)[idx]);
    if (w_dtype == 2) return oracle_e4m3_decode(((const uint8_t *)w)[idx]);
    uint8_t b = ((const uint8_t *)w)[idx / 2];
    uint8_t nib = (col & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
    uint8_t sc = ((const uint8_t *)wscale)[row * (size_t)(len / 32) + (size_t)(col / 32)];
    return e2m1_table[nib] * e8m0_table[sc];
}

int oracle_expert_ffn(int T, int K, int E, int H, int I, int w_dtype, int x_dtype, int inter,
                      const void *x, const void *w13, const void *w13_scale,
                      const void *w2, const void *w2_scale,
                      const int32_t *topk_ids, float *y_slots)
{
    if (T < 0 || K < 1 || E < 1 || H < 1 || I < 1) return 1;
    if (w_dtype < 0 || w_dtype > 3) return 1;
    if (w_dtype >= 2 && x_dtype != 1) return 1;
    if (w_dtype >= 2 && (!w13_scale || !w2_scale)) return 1;
    if (w_dtype == 3 && (H % 32 || I % 32)) return 1;
    mx_tables();
    const float *s13 = (const float *)w13_scale, *s2 = (const float *)w2_scale;
    int64_t S = (int64_t)T * K;
    uint8_t *xq = NULL;
    float *sx = NULL;
    if (w_dtype >= 2) {
        xq = (uint8_t *)malloc((size_t)T * H);
        sx = (float *)malloc(sizeof(float) * (size_t)T);
        oracle_quant_tokens_e4m3((const uint16_t *)x, T, H, xq, sx);
    }
    int err = 0;
#pragma omp parallel
    {
        double *xt = (double *)malloc(sizeof(double) * (size_t)H);
        double *a = (double *)malloc(sizeof(double) * (size_t)I);
        float *a32 = (float *)malloc(sizeof(float) * (size_t)I);
        uint8_t *aq = (uint8_t *)malloc((size_t)I);
        if (!xt || !a || !a32 || !aq) err = 1;
#pragma omp for schedule(dynamic)
        for (int64_t i = 0; i < S; i++) {
            int t = (int)(i / K);
            int e = topk_ids[i];
            if (e < 0 || e >= E || !xt || !a || !a32 || !aq) continue;
            /* the token's activations */
            for (int h = 0; h < H; h++) {
                size_t xi = (size_t)t * H + h;
                if (w_dtype >= 2) xt[h] = oracle_e4m3_decode(xq[xi]);
                else if (x_dtype == 0) xt[h] = (double)((const float *)x)[xi];
                else xt[h] = oracle_bf16_decode(((const uint16_t *)x)[xi]);
            }
            /* gate and up projections, SiLU(gate) * up */
            for (int j = 0; j < I; j++) {
                size_t rg = (size_t)e * 2 * I + j;          /* rows of W13 */
                size_t ru = (size_t)e * 2 * I + I + j;
                double g = 0.0, u = 0.0;
                for (int h = 0; h < H; h++) {
                    g += xt[h] * load_w(w_dtype, w13, w13_scale, rg, h, H);
                    u += xt[h] * load_w(w_dtype, w13, w13_scale, ru, h, H);
                }
                if (w_dtype == 2) {
                    g = g * (double)sx[t] * (double)s13[rg];
                    u = u * (double)sx[t] * (double)s13[ru];
                } else if (w_dtype == 3) {                 /* block scales are in the values */
                    g = g * (double)sx[t];
                    u = u * (double)sx[t];
                }
                a[j] = g / (1.0 + exp(-g)) * u;
            }
            /* the intermediate's type */
            double sa = 1.0;
            for (int j = 0; j < I; j++) a32[j] = (float)a[j];
            if (inter == 1) {
                for (int j = 0; j < I; j++) a[j] = (double)a32[j];
            } else if (inter == 2) {
                for (int j = 0; j < I; j++) a[j] = oracle_bf16_decode(oracle_bf16_encode(a32[j]));
            } else if (inter == 3) {
                float s_row;
                oracle_quant_row_e4m3(a32, I, aq, &s_row);
                for (int j = 0; j < I; j++) a[j] = oracle_e4m3_decode(aq[j]);
                sa = (double)s_row;
            }
            /* down projection */
            for (int h = 0; h < H; h++) {
                size_t rd = (size_t)e * H + h;              /* row of W2 */
                double y = 0.0;
                for (int j = 0; j < I; j++) y += a[j] * load_w(w_dtype, w2, w2_scale, rd, j, I);
                if (w_dtype == 2) y = y * sa * (double)s2[rd];
                else if (inter == 3) y = y * sa;
                y_slots[i * H + h] = (float)y;
            }
        }
        free(xt); free(a); free(a32); free(aq);
    }
    free(xq); free(sx);
    return err;
}

/*
 * Top-k weighted combine.  [DIG] opening paragraphs: the layer's output for a
 * token is the gate-weighted result of its chosen experts' FFNs; [GCM]: the
 * shared expert joins the sum (here it is the appended last column, weight 1).
 *   out[t,h] = sum_{k=0..K-1, ids[t,k] in [0,E)} w[t,k] * y_slots[t*K+k, h]
 * summed in double in ascending k.
 */
int oracle_combine(int T, int K, int E, int H, const float *y_slots,
                   const float *topk_weights, const int32_t *topk_ids, double *out)
{
    if (T < 0 || K < 1 || H < 1) return 1;
    for (int t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) {
            double acc = 0.0;
            for (int k = 0; k < K; k++) {
                int64_t i = (int64_t)t * K + k;
                int e = topk_ids[i];
                if (e < 0 || e >= E) continue;
                acc += (double)topk_weights[i] * (double)y_slots[i * H + h];
            }
            out[(size_t)t * H + h] = acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Permute / unpermute around the grouped FFN                                */
/* ------------------------------------------------------------------------ */
/*
 * [DIG] opening paragraphs, the TransformerEngine paragraph and its "MoE
 * Permute example" figure: besides ordering token slots by expert, a permute
 * step moves the rows and records where each source row went; the reverse
 * movement (unpermute) is its gradient.  [GCM] abstract: under expert
 * parallelism a layer pays a token dispatch, the grouped GEMMs and a combine.
 * Reading: the destination order is Align & Sort's padded layout, so every
 * expert's rows are contiguous (one contiguous send range per destination
 * GPU); padding rows are zero; rows from P = num_tokens_post_padded on hold
 * no expert's data and are left as they were.
 *   x_perm[r]      = x[sorted[r] / K]   (r < P, sorted[r] < S), else zeros (r < P)
 *   row_of_slot[i] = the r with sorted[r] = i, or -1 if slot i is not placed
 *   out[t]         = sum over k ascending of w[t,k] * y_perm[row_of_slot[t*K+k]],
 *                    slots with row -1 skipped, in double
 */
int oracle_permute_rows(const uint8_t *x, int T, int64_t row_bytes, int K, const int32_t *sorted,
                        int64_t P, uint8_t *x_perm)
{
    if (T < 0 || K < 1 || row_bytes < 0 || P < 0) return 1;
    int64_t S = (int64_t)T * K;
    for (int64_t r = 0; r < P; r++) {
        uint8_t *dst = x_perm + r * row_bytes;
        if (sorted[r] >= 0 && sorted[r] < S)
            memcpy(dst, x + (int64_t)(sorted[r] / K) * row_bytes, (size_t)row_bytes);
        else
            memset(dst, 0, (size_t)row_bytes);
    }
    return 0;
}

int oracle_row_of_slot(const int32_t *sorted, int64_t C, int64_t S, int32_t *row_of_slot)
{
    if (C < 0 || S < 0) return 1;
    for (int64_t i = 0; i < S; i++) row_of_slot[i] = -1;
    for (int64_t r = 0; r < C; r++)
        if (sorted[r] >= 0 && sorted[r] < S) row_of_slot[sorted[r]] = (int32_t)r;
    return 0;
}

int oracle_unpermute_combine(int T, int K, int H, const float *y_perm, const float *topk_weights,
                             const int32_t *row_of_slot, double *out)
{
    if (T < 0 || K < 1 || H < 1) return 1;
    for (int t = 0; t < T; t++)
        for (int h = 0; h < H; h++) {
            double acc = 0.0;
            for (int k = 0; k < K; k++) {
                int64_t i = (int64_t)t * K + k;
                int32_t r = row_of_slot[i];
                if (r < 0) continue;
                acc += (double)topk_weights[i] * (double)y_perm[(int64_t)r * H + h];
            }
            out[(size_t)t * H + h] = acc;
        }
    return 0;
}

/* Gradient of the unpermute-combine for an upstream d_out [T,H] ([DIG], the
 * Megatron section: permute and unpermute are each other's gradients, so the
 * gradient of the weighted unpermute is a weighted permute).  out is linear
 * in both y_perm and w, so, in double:
 *   d_y_perm[r] = w[s] * d_out[s / K]     for r < P, s = sorted[r] < S;
 *                 zeros for a padding row r < P (no slot reads it)
 *   d_w[s]      = sum_h d_out[s / K, h] * y_perm[row of s, h]; 0 for a slot
 *                 that is not placed (its id was outside [0,E))
 * round: how d_y_perm is delivered -- 0 exact (the product of two floats is
 * exact in double), 1 rounded to fp32, 2 rounded to fp32 then to bf16 (the
 * reading: the product is formed in fp32 and rounded once more to the output
 * type).  Rows from P on are not written. */
int oracle_unpermute_combine_backward(int T, int K, int H, const float *d_out, const float *y_perm,
                                      const float *topk_weights, const int32_t *sorted, int64_t P,
                                      int round, double *d_y_perm, double *d_w)
{
    if (T < 0 || K < 1 || H < 1 || P < 0 || round < 0 || round > 2) return 1;
    int64_t S = (int64_t)T * K;
    for (int64_t i = 0; i < S; i++) d_w[i] = 0.0;
    for (int64_t r = 0; r < P; r++) {
        double *dst = d_y_perm + r * H;
        int32_t s = sorted[r];
        if (s < 0 || s >= S) {
            for (int h = 0; h < H; h++) dst[h] = 0.0;
            continue;
        }
        const float *g = d_out + (int64_t)(s / K) * H;
        const float *y = y_perm + r * H;
        double dot = 0.0;
        for (int h = 0; h < H; h++) {
            double v = (double)topk_weights[s] * (double)g[h];
            if (round >= 1) v = (double)(float)v;
            if (round == 2) v = oracle_bf16_decode(oracle_bf16_encode((float)v));
            dst[h] = v;
            dot += (double)g[h] * (double)y[h];
        }
        d_w[s] = dot;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward (training)                                                        */
/* ------------------------------------------------------------------------ */
/*
 * [DIG] the Megatron section (for training, the permute gets its gradient
 * operation, unpermute) and the TransformerEngine paragraph; [XMOE] abstract
 * (MoE training on AMD GPUs).  The pages give no formulas, so the backward is
 * the exact derivative of the forward above, in double:
 *   d_w[t,k]   = sum_h d_out[t,h] * y_slots[t*K+k,h]      (the forward's y)
 *   d_y        = w[t,k] * d_out[t]
 *   dW2[e,h,j] += d_y[h] * a~_j       a~ = the intermediate as the forward
 *                                      rounds it (inter 0: none, 2: bf16)
 *   d_a_j      = sum_h d_y[h] * W2[e,h,j]   (the rounding passed straight
 *                                             through: d a~ / d a = 1)
 *   d_g_j      = d_a_j * u_j * SiLU'(g_j),  SiLU'(g) = s(g) (1 + g (1 - s(g)))
 *   d_u_j      = d_a_j * SiLU(g_j)
 *   dW13[e,j,h] += d_g_j x_h,  dW13[e,I+j,h] += d_u_j x_h
 *   dx[t,h]    += sum_j d_g_j W13[e,j,h] + d_u_j W13[e,I+j,h]
 * over every slot with an id in [0,E).  fp32 or bf16 weights and activations
 * (w_dtype = x_dtype 0 or 1), decoded exactly.  Outputs are overwritten.
 */
int oracle_ffn_backward(int T, int K, int E, int H, int I, int w_dtype, int x_dtype, int inter,
                        const void *x, const void *w13, const void *w2, const int32_t *topk_ids,
                        const float *topk_weights, const float *y_slots, const float *d_out,
                        double *dx, double *dw13, double *dw2, double *d_w)
{
    if (T < 0 || K < 1 || E < 1 || H < 1 || I < 1) return 1;
    if (w_dtype < 0 || w_dtype > 1 || x_dtype < 0 || x_dtype > 1) return 1;
    if (inter != 0 && inter != 2) return 1;
    int64_t S = (int64_t)T * K;
    /* per slot: the forward's intermediate and the slot's gradient vectors */
    double *xd = (double *)malloc(sizeof(double) * (size_t)T * H);
    double *at = (double *)calloc((size_t)S * I, sizeof(double));
    double *dg = (double *)calloc((size_t)S * I, sizeof(double));
    double *du = (double *)calloc((size_t)S * I, sizeof(double));
    double *dy = (double *)calloc((size_t)S * H, sizeof(double));
    if (!xd || !at || !dg || !du || !dy) { free(xd); free(at); free(dg); free(du); free(dy); return 1; }
    for (int64_t q = 0; q < (int64_t)T * H; q++)
        xd[q] = x_dtype == 0 ? (double)((const float *)x)[q] : oracle_bf16_decode(((const uint16_t *)x)[q]);
#pragma omp parallel
    {
        double *g = (double *)malloc(sizeof(double) * (size_t)I);
        double *u = (double *)malloc(sizeof(double) * (size_t)I);
        double *da = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic)
        for (int64_t i = 0; i < S; i++) {
            int t = (int)(i / K);
            int e = topk_ids[i];
            d_w[i] = 0.0;
            if (e < 0 || e >= E) continue;
            const double *xt = xd + (size_t)t * H;
            double dwi = 0.0;
            for (int h = 0; h < H; h++) dwi += (double)d_out[(size_t)t * H + h] * (double)y_slots[i * H + h];
            d_w[i] = dwi;
            for (int h = 0; h < H; h++) dy[i * H + h] = (double)topk_weights[i] * (double)d_out[(size_t)t * H + h];
            for (int j = 0; j < I; j++) {
                size_t rg = (size_t)e * 2 * I + j, ru = rg + I;
                double gj = 0.0, uj = 0.0;
                for (int h = 0; h < H; h++) {
                    gj += xt[h] * load_w(w_dtype, w13, NULL, rg, h, H);
                    uj += xt[h] * load_w(w_dtype, w13, NULL, ru, h, H);
                }
                g[j] = gj;
                u[j] = uj;
                double a = gj / (1.0 + exp(-gj)) * uj;
                at[i * I + j] = inter == 2 ? oracle_bf16_decode(oracle_bf16_encode((float)a)) : a;
                da[j] = 0.0;
            }
            for (int h = 0; h < H; h++)
                for (int j = 0; j < I; j++)
                    da[j] += dy[i * H + h] * load_w(w_dtype, w2, NULL, (size_t)e * H + h, j, I);
            for (int j = 0; j < I; j++) {
                double sg = 1.0 / (1.0 + exp(-g[j]));
                dg[i * I + j] = da[j] * u[j] * sg * (1.0 + g[j] * (1.0 - sg));
                du[i * I + j] = da[j] * g[j] * sg;
            }
        }
        free(g); free(u); free(da);
    }
    /* weight gradients: each element summed over the expert's slots in ascending order */
#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < (int64_t)E * H; r++) {
        int e = (int)(r / H), h = (int)(r % H);
        double *out = dw2 + (size_t)r * I;
        for (int j = 0; j < I; j++) out[j] = 0.0;
        for (int64_t i = 0; i < S; i++) {
            if (topk_ids[i] != e) continue;
            for (int j = 0; j < I; j++) out[j] += dy[i * H + h] * at[i * I + j];
        }
    }
#pragma omp parallel for schedule(dynamic)
    for (int64_t r = 0; r < (int64_t)E * 2 * I; r++) {
        int e = (int)(r / (2 * I)), j = (int)(r % (2 * I));
        const double *src = j < I ? dg : du;
        int jj = j < I ? j : j - I;
        double *out = dw13 + (size_t)r * H;
        for (int h = 0; h < H; h++) out[h] = 0.0;
        for (int64_t i = 0; i < S; i++) {
            if (topk_ids[i] != e) continue;
            const double *xt = xd + (size_t)(i / K) * H;
            for (int h = 0; h < H; h++) out[h] += src[i * I + jj] * xt[h];
        }
    }
    /* the activations' gradient: slots in ascending k, then j */
#pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < T; t++) {
        double *out = dx + (size_t)t * H;
        for (int h = 0; h < H; h++) out[h] = 0.0;
        for (int k = 0; k < K; k++) {
            int64_t i = (int64_t)t * K + k;
            int e = topk_ids[i];
            if (e < 0 || e >= E) continue;
            for (int j = 0; j < I; j++) {
                size_t rg = (size_t)e * 2 * I + j, ru = rg + I;
                for (int h = 0; h < H; h++)
                    out[h] += dg[i * I + j] * load_w(w_dtype, w13, NULL, rg, h, H) +
                              du[i * I + j] * load_w(w_dtype, w13, NULL, ru, h, H);
            }
        }
    }
    free(xd); free(at); free(dg); free(du); free(dy);
    return 0;
}

/*
 * Routing backward: d_logits [T,E] from d_w [T,K], the selection held fixed
 * (it is piecewise constant in the logits; the bias only selects).  With
 * s_e = softmax(logits)_e or sigmoid(logits_e) in double, the forward's
 * weights of the routed columns are w_k = c * s_{e_k} / N, c = routed_scaling,
 * N = the sum of s over the chosen experts when renormalising, else 1.  An
 * appended shared column (id E, weight 1) has no gradient.
 *   dL/ds_e = c * (d_w_k / N - [renormalise] sum_j d_w_j s_{e_j} / N^2)  for e = e_k
 *   softmax: d l_i = s_i (dL/ds_i - sum_e dL/ds_e s_e);  sigmoid: d l_i = dL/ds_i s_i (1 - s_i)
 */
int oracle_route_backward(int T, int E, int K, int score_mode, int renormalize, double routed_scaling,
                          int append_shared, const float *logits, const int32_t *topk_ids,
                          const float *d_w, double *d_logits)
{
    if (T < 0 || E < 1 || K < 1) return 1;
    int KO = K + (append_shared ? 1 : 0);
    double *s = (double *)malloc(sizeof(double) * (size_t)E);
    double *gs = (double *)malloc(sizeof(double) * (size_t)E);
    for (int t = 0; t < T; t++) {
        const float *l = logits + (size_t)t * E;
        if (score_mode == 0) {
            double mx = -INFINITY, z = 0.0;
            for (int e = 0; e < E; e++) if ((double)l[e] > mx) mx = (double)l[e];
            for (int e = 0; e < E; e++) { s[e] = exp((double)l[e] - mx); z += s[e]; }
            for (int e = 0; e < E; e++) s[e] /= z;
        } else {
            for (int e = 0; e < E; e++) s[e] = 1.0 / (1.0 + exp(-(double)l[e]));
        }
        double N = 1.0, sdw = 0.0;
        if (renormalize) {
            N = 0.0;
            for (int k = 0; k < K; k++) N += s[topk_ids[(size_t)t * KO + k]];
        }
        for (int k = 0; k < K; k++)
            sdw += (double)d_w[(size_t)t * KO + k] * s[topk_ids[(size_t)t * KO + k]];
        for (int e = 0; e < E; e++) gs[e] = 0.0;
        for (int k = 0; k < K; k++) {
            int e = topk_ids[(size_t)t * KO + k];
            double v = (double)d_w[(size_t)t * KO + k] / N;
            if (renormalize) v -= sdw / (N * N);
            gs[e] += routed_scaling * v;
        }
        double *dl = d_logits + (size_t)t * E;
        if (score_mode == 0) {
            double dot = 0.0;
            for (int e = 0; e < E; e++) dot += gs[e] * s[e];
            for (int e = 0; e < E; e++) dl[e] = s[e] * (gs[e] - dot);
        } else {
            for (int e = 0; e < E; e++) dl[e] = gs[e] * s[e] * (1.0 - s[e]);
        }
    }
    free(s); free(gs);
    return 0;
}
