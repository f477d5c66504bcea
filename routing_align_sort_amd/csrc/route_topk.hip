// Top-k expert routing for gfx950: one wave per token.
//
// What it computes is set by "AMD GPU ... 7x faster ... efficient MoE with any
// number of experts" (dignews.cc), opening paragraphs and FasterTransformer
// section: top-K gating over softmax scores, and the biased variant of
// DeepSeek V3/R1 where a per-expert bias steers the choice.  The group limit
// (n_group / topk_group) is DeepSeek-V3's rule, which the page cites but does
// not spell out; the exact rule is in include/moe_mi355x.h.
//
// Precision: scores are formed in double and rounded once to fp32, so every
// fp32 key the selection compares is the correctly rounded image of the
// score; keys and group scores are single fp32 additions.  Weights use the
// double scores.
#include "common.hpp"
#include "kernels.hpp"
#include "quant.hpp"

namespace moe {

constexpr int kRouteWaves = 4;
constexpr int kRouteMaxPerLane = kRouteMaxExperts / kWave;   // 16

// A candidate as one ordered 64-bit word: the fp32 key mapped to an unsigned
// integer of the same order in the high half, and ~e in the low half, so the
// largest word is the largest key and, among equal keys, the lowest id.
// 0 = no candidate (every real word is larger).
__device__ __forceinline__ uint64_t cand_word(float key, int e) {
    const uint32_t b = __float_as_uint(key);
    const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)k << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int cand_id(uint64_t w) { return (int)(0xFFFFFFFFu - (uint32_t)w); }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t d = __shfl_xor(v, o, kWave);
        v = d > v ? d : v;
    }
    return v;
}

// JT: experts per lane the loops are unrolled for (a power of two with
// 64*JT >= E), so a token of E experts does E/64 lanes' worth of work, not
// the 1024-expert maximum's.
template <int JT>
__device__ __forceinline__ void route_token_block(const RouteArgs& a, int block) {
    __shared__ float keys_lds[kRouteWaves][kRouteMaxExperts];
    const int w = threadIdx.x / kWave;
    const int lane = lane_id();
    const int t = block * kRouteWaves + w;
    if (t >= a.T) return;                       // whole wave leaves; no block barriers below
    const int E = a.E;
    static_assert(JT <= kRouteMaxPerLane && JT <= 32, "experts per lane");
    const float* lg = a.logits + (int64_t)t * E;

    float key[JT];
    double sc[JT];
    // 1. scores in double
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < JT; ++j) {
        const int e = lane + j * kWave;
        key[j] = (e < E) ? lg[e] : -INFINITY;
        m = fmaxf(m, key[j]);
    }
    if (a.score == 0) {
        m = wave_max_f32(m);
        double z = 0.0;
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int e = lane + j * kWave;
            sc[j] = (e < E) ? exp((double)key[j] - (double)m) : 0.0;
            z += sc[j];
        }
        z = wave_sum_f64(z);
#pragma unroll
        for (int j = 0; j < JT; ++j) sc[j] = sc[j] / z;
    } else {
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int e = lane + j * kWave;
            sc[j] = (e < E) ? 1.0 / (1.0 + exp(-(double)key[j])) : 0.0;
        }
    }
    // 2. selection keys in fp32
    uint32_t allowed = 0;
#pragma unroll
    for (int j = 0; j < JT; ++j) {
        const int e = lane + j * kWave;
        if (e < E) {
            const float s32 = (float)sc[j];
            key[j] = a.bias ? s32 + a.bias[e] : s32;
            allowed |= 1u << j;
        }
    }
    // 3. group limit
    if (a.n_group > 1) {
        const int gsize = E / a.n_group;
        float gs = -INFINITY;                       // lane g (< n_group): group g's score
        if ((gsize & (gsize - 1)) == 0 && gsize <= kWave) {
            // a group is an aligned run of gsize lanes of one register: its
            // two largest keys by a butterfly over the run, then each lane g
            // fetches its group's sum from the run's first lane
            float gsum[JT];
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                float b1 = key[j], b2 = -INFINITY;
                for (int o = gsize >> 1; o > 0; o >>= 1) {
                    const float c1 = __shfl_xor(b1, o, kWave), c2 = __shfl_xor(b2, o, kWave);
                    b2 = fmaxf(fminf(b1, c1), fmaxf(b2, c2));
                    b1 = fmaxf(b1, c1);
                }
                gsum[j] = gsize >= 2 ? b1 + b2 : b1;
            }
            const int first = lane * gsize;          // group `lane`'s first expert
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                const float v = __shfl(gsum[j], first & (kWave - 1), kWave);
                if (lane < a.n_group && (first >> 6) == j) gs = v;
            }
        } else {
#pragma unroll
            for (int j = 0; j < JT; ++j) {
                const int e = lane + j * kWave;
                if (e < E) keys_lds[w][e] = key[j];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // lane g scores group g: the sum of its two largest keys
            if (lane < a.n_group) {
                float b1 = -INFINITY, b2 = -INFINITY;
                int n = 0;
                for (int e = lane * gsize; e < (lane + 1) * gsize; ++e) {
                    const float k = keys_lds[w][e];
                    if (n == 0 || k > b1) { b2 = b1; b1 = k; }
                    else if (n == 1 || k > b2) { b2 = k; }
                    ++n;
                }
                gs = (gsize >= 2) ? b1 + b2 : b1;
            }
        }
        // the topk_group best groups (higher score, lower index on ties)
        uint64_t gw = lane < a.n_group ? cand_word(gs, lane) : 0;
        bool keep = false;
        for (int r = 0; r < a.topk_group; ++r) {
            const uint64_t best = wave_max_u64(keep ? 0 : gw);
            if (cand_id(best) == lane) keep = true;
        }
        const uint64_t kept = ballot(keep);
        uint32_t al = 0;
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int e = lane + j * kWave;
            if (e < E && ((kept >> (e / gsize)) & 1ull)) al |= 1u << j;
        }
        allowed = al;
    }
    // 4. top-K, one wave-wide maximum of candidate words per pick (descending
    //    order, lower id on ties); the winner's double score comes from its lane
    double my_s = 0.0, sum = 0.0;
    int my_e = 0;
    for (int k = 0; k < a.K; ++k) {
        uint64_t c = 0;
#pragma unroll
        for (int j = 0; j < JT; ++j)
            if ((allowed >> j) & 1u) {
                const uint64_t d = cand_word(key[j], lane + j * kWave);
                c = d > c ? d : c;
            }
        const int be = cand_id(wave_max_u64(c));
        const int bj = be / kWave;
        double s_b = 0.0;
#pragma unroll
        for (int j = 0; j < JT; ++j)
            if (j == bj) s_b = sc[j];
        s_b = __shfl(s_b, be & (kWave - 1), kWave);
        if ((be & (kWave - 1)) == lane) allowed &= ~(1u << bj);
        sum += s_b;                               // ascending k, as the definition sums
        if (lane == k) { my_s = s_b; my_e = be; }
    }
    // 5. weights
    const int KO = a.K + (a.append_shared ? 1 : 0);
    if (lane < a.K) {
        double wt = my_s;
        if (a.renormalize) wt = wt / sum;
        wt = wt * (double)a.routed_scaling;
        a.topk_ids[(int64_t)t * KO + lane] = my_e;
        a.topk_weights[(int64_t)t * KO + lane] = (float)wt;
    }
    if (a.append_shared && lane == 0) {
        a.topk_ids[(int64_t)t * KO + a.K] = E;
        a.topk_weights[(int64_t)t * KO + a.K] = 1.0f;
    }
}

template <int JT>
__global__ void __launch_bounds__(kRouteWaves* kWave)
route_topk_kernel(RouteArgs a) {
    route_token_block<JT>(a, blockIdx.x);
}

// Routing and the per-token activation quantisation in one launch: the
// first ceil(T/4) workgroups route four tokens each, the next T quantise one
// token row each.  The two jobs are independent (both read their own inputs
// only), so one launch runs them side by side instead of one after the other.
static_assert(kQuantThreads == kRouteWaves * kWave, "one workgroup size for both jobs");
template <int JT>
__global__ void __launch_bounds__(kRouteWaves* kWave)
route_quant_kernel(RouteArgs a, QuantArgs q) {
    const int nr = (a.T + kRouteWaves - 1) / kRouteWaves;
    if ((int)blockIdx.x < nr)
        route_token_block<JT>(a, blockIdx.x);
    else
        quant_token_row(q.x, q.H, q.xq, q.sx, q.amax, q.C, (int)blockIdx.x - nr, (int)gridDim.x - nr);
}

hipError_t launch_route_quant(const RouteArgs& a, const QuantArgs& q, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int blocks = (a.T + kRouteWaves - 1) / kRouteWaves + a.T;
    const int J = (a.E + kWave - 1) / kWave;
    const dim3 g(blocks), b(kRouteWaves * kWave);
    if (J <= 1) hipLaunchKernelGGL(route_quant_kernel<1>, g, b, 0, stream, a, q);
    else if (J <= 2) hipLaunchKernelGGL(route_quant_kernel<2>, g, b, 0, stream, a, q);
    else if (J <= 4) hipLaunchKernelGGL(route_quant_kernel<4>, g, b, 0, stream, a, q);
    else if (J <= 8) hipLaunchKernelGGL(route_quant_kernel<8>, g, b, 0, stream, a, q);
    else if (J <= kRouteMaxPerLane) hipLaunchKernelGGL(route_quant_kernel<kRouteMaxPerLane>, g, b, 0, stream, a, q);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_route_topk(const RouteArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int blocks = (a.T + kRouteWaves - 1) / kRouteWaves;
    const int J = (a.E + kWave - 1) / kWave;
    const dim3 g(blocks), b(kRouteWaves * kWave);
    if (J <= 1) hipLaunchKernelGGL(route_topk_kernel<1>, g, b, 0, stream, a);
    else if (J <= 2) hipLaunchKernelGGL(route_topk_kernel<2>, g, b, 0, stream, a);
    else if (J <= 4) hipLaunchKernelGGL(route_topk_kernel<4>, g, b, 0, stream, a);
    else if (J <= 8) hipLaunchKernelGGL(route_topk_kernel<8>, g, b, 0, stream, a);
    else if (J <= kRouteMaxPerLane) hipLaunchKernelGGL(route_topk_kernel<kRouteMaxPerLane>, g, b, 0, stream, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
