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

namespace moe {

constexpr int kRouteWaves = 4;
constexpr int kRouteMaxPerLane = kRouteMaxExperts / kWave;   // 16

struct Cand {
    float key;
    int e;          // INT32_MAX = none
    double s;
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
    if (a.e == INT32_MAX) return false;
    if (b.e == INT32_MAX) return true;
    return a.key > b.key || (a.key == b.key && a.e < b.e);
}

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        Cand d;
        d.key = __shfl_xor(c.key, o, kWave);
        d.e = __shfl_xor(c.e, o, kWave);
        d.s = __shfl_xor(c.s, o, kWave);
        if (better(d, c)) c = d;
    }
    return c;
}

// JT: experts per lane the loops are unrolled for (a power of two with
// 64*JT >= E), so a token of E experts does E/64 lanes' worth of work, not
// the 1024-expert maximum's.
template <int JT>
__global__ void __launch_bounds__(kRouteWaves* kWave)
route_topk_kernel(RouteArgs a) {
    __shared__ float keys_lds[kRouteWaves][kRouteMaxExperts];
    const int w = threadIdx.x / kWave;
    const int lane = lane_id();
    const int t = blockIdx.x * kRouteWaves + w;
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
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int e = lane + j * kWave;
            if (e < E) keys_lds[w][e] = key[j];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane g scores group g: the sum of its two largest keys
        Cand g{-INFINITY, INT32_MAX, 0.0};
        if (lane < a.n_group) {
            float b1 = -INFINITY, b2 = -INFINITY;
            int n = 0;
            for (int e = lane * gsize; e < (lane + 1) * gsize; ++e) {
                const float k = keys_lds[w][e];
                if (n == 0 || k > b1) { b2 = b1; b1 = k; }
                else if (n == 1 || k > b2) { b2 = k; }
                ++n;
            }
            g.key = (gsize >= 2) ? b1 + b2 : b1;
            g.e = lane;
        }
        bool keep = false;
        for (int r = 0; r < a.topk_group; ++r) {
            Cand c = g;
            if (keep) c.e = INT32_MAX;
            const Cand best = wave_best(c);
            if (best.e == lane) keep = true;
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
    // 4. top-K, one wave-wide argmax per pick (descending order, lower id on ties)
    double my_s = 0.0, sum = 0.0;
    int my_e = 0;
    for (int k = 0; k < a.K; ++k) {
        Cand c{-INFINITY, INT32_MAX, 0.0};
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            if ((allowed >> j) & 1u) {
                const Cand d{key[j], lane + j * kWave, sc[j]};
                if (better(d, c)) c = d;
            }
        }
        const Cand best = wave_best(c);
        if ((best.e & (kWave - 1)) == lane) allowed &= ~(1u << (best.e / kWave));
        sum += best.s;                            // ascending k, as the definition sums
        if (lane == k) { my_s = best.s; my_e = best.e; }
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
