// MoE Align & Sort for gfx950.
//
// What it computes is set by "AMD GPU ... 7x faster ... efficient MoE with any
// number of experts" (dignews.cc): the opening paragraphs (order token slots by
// expert id, each expert's run padded to whole blocks of block_size_m) and the
// section on the three-part algorithm (distributed concurrent counting, cumsum
// with local / merged / aligned stages, parallel placement).  The result is a
// stable counting sort; see include/moe_mi355x.h for the exact outputs.
//
// Design on MI355X
// ----------------
// * Ranks come from wave ballots, not atomics: for each 64-slot step a wave
//   builds, per lane, the mask of lanes holding the same expert from one
//   ballot per id bit; the lane's rank is the popcount of that mask below it
//   and the lowest lane adds the step's count to the wave's running LDS
//   counter.  Waves own contiguous sub-chunks, so (workgroup base + wave base
//   + running count) is the stable position; placement needs no atomics.
// * Small inputs run as ONE workgroup of 1024 threads and one launch:
//   count -> per-wave prefix -> aligned scan over experts -> placement.
// * Large inputs run as G workgroups (G a multiple of the XCD count, 8) in two
//   launches.  Launch 1 counts each workgroup's contiguous chunk into a
//   [G,E] matrix in the workspace.  Launch 2 is the merge + aligned cumsum +
//   placement: every workgroup reads the small matrix, forms its own per-
//   expert base and the global aligned offsets (redundantly, which costs one
//   small L2 read instead of a grid-wide barrier across dies), recounts its
//   chunk per wave and scatters.  Padding, the tail and expert_ids are
//   written by all workgroups in a grid-strided pattern.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

// Mask of the lanes whose valid expert id equals this lane's.
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool valid, int nbits) {
    uint64_t peers = ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

// One wave walks slots [s0, s1) in 64-slot steps.  Count mode adds each
// expert's occurrences to run[e]; place mode writes slot i to
// sorted[run[e] + rank] and advances run[e].  run[] is this wave's LDS row.
template <bool kPlace>
__device__ __forceinline__ void walk_slots(const int32_t* __restrict__ ids, int64_t s0, int64_t s1,
                                           int E, int nbits, int* run, int32_t* __restrict__ sorted) {
    const int lane = lane_id();
    for (int64_t base = s0; base < s1; base += kWave) {
        const int64_t i = base + lane;
        const int e = (i < s1) ? ids[i] : -1;
        const bool valid = (e >= 0) && (e < E);
        const uint64_t peers = same_expert_lanes(valid ? e : 0, valid, nbits);
        if (valid) {
            const int r = popc_below(peers);
            const int n = __popcll(peers);
            if (kPlace) {
                const int pos = run[e];
                sorted[pos + r] = (int32_t)i;
                if (r == 0) run[e] = pos + n;
            } else {
                if (r == 0) run[e] += n;
            }
        }
    }
}

// Slots of a workgroup chunk [c0,c1) owned by wave w (64-aligned sub-chunks).
__device__ __forceinline__ void wave_range(int64_t c0, int64_t c1, int w, int64_t* s0, int64_t* s1) {
    const int64_t len = c1 - c0;
    int64_t sub = (len + kAlignWaves - 1) / kAlignWaves;
    sub = (sub + kWave - 1) / kWave * kWave;
    int64_t a = c0 + (int64_t)w * sub;
    int64_t b = a + sub;
    if (a > c1) a = c1;
    if (b > c1) b = c1;
    *s0 = a;
    *s1 = b;
}

// Exclusive prefix sum over the 1024 threads of a workgroup; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* lds16, int* total) {
    const int w = threadIdx.x / kWave;
    const int incl = wave_incl_scan_i32(v);
    if (lane_id() == kWave - 1) lds16[w] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kAlignWaves; ++i) {
        const int t = lds16[i];
        before += (i < w) ? t : 0;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// Largest e with off[e] <= p (off non-decreasing, off[0] = 0 <= p < off[E]).
__device__ __forceinline__ int find_expert(const int* off, int E, int64_t p) {
    int lo = 0, hi = E;            // off[lo] <= p < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)off[mid] <= p) lo = mid; else hi = mid;
    }
    return lo;
}

struct AlignOut {
    int32_t* sorted;
    int32_t* expert_ids;
    int32_t* post_padded;
    int32_t* offsets;
};

// Writes everything that depends only on the aligned offsets: P, offsets,
// expert_ids, the padding inside every expert's run and the tail [P, C).
// gthread/gstride spread the work over the whole grid.
__device__ void write_layout(const AlignOut& o, const int* off, const int* total, int E, int B,
                             int64_t S, int64_t C, int64_t gthread, int64_t gstride) {
    const int P = off[E];
    if (gthread == 0) o.post_padded[0] = P;
    if (o.offsets)
        for (int64_t e = gthread; e <= E; e += gstride) o.offsets[e] = off[e];
    const int64_t nblk = C / B;
    for (int64_t j = gthread; j < nblk; j += gstride) {
        const int64_t p = j * B;
        o.expert_ids[j] = (p < P) ? find_expert(off, E, p) : -1;
    }
    for (int64_t e = gthread; e < E; e += gstride)
        for (int64_t p = off[e] + total[e]; p < off[e + 1]; ++p) o.sorted[p] = (int32_t)S;
    for (int64_t p = P + gthread; p < C; p += gstride) o.sorted[p] = (int32_t)S;
}

// LDS: hist[kAlignWaves][E], off[E+1], total[E], scan scratch[16].
__host__ __device__ inline size_t align_lds_ints(int E) {
    return (size_t)kAlignWaves * E + (E + 1) + E + 16;
}

// ---------------------------------------------------------------- 1 launch --
__global__ void __launch_bounds__(kAlignThreads)
align_single_kernel(const int32_t* __restrict__ ids, int64_t S, int E, int B, int nbits, int64_t C,
                    AlignOut o) {
    extern __shared__ int lds[];
    int* hist = lds;                               // [waves][E]
    int* off = hist + kAlignWaves * E;             // [E+1]
    int* total = off + E + 1;                      // [E]
    int* scr = total + E;                          // [16]
    const int tid = threadIdx.x, w = tid / kWave;
    for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) hist[i] = 0;
    __syncthreads();

    int64_t s0, s1;
    wave_range(0, S, w, &s0, &s1);
    walk_slots<false>(ids, s0, s1, E, nbits, hist + w * E, nullptr);
    __syncthreads();

    // per expert: exclusive prefix over waves, and the total
    int padded = 0;
    for (int e = tid; e < E; e += kAlignThreads) {
        int run = 0;
        for (int v = 0; v < kAlignWaves; ++v) {
            const int c = hist[v * E + e];
            hist[v * E + e] = run;
            run += c;
        }
        total[e] = run;
        padded = (run + B - 1) / B * B;            // E <= 1024: one expert per thread
    }
    int sum;
    const int ex = block_excl_scan(tid < E ? padded : 0, scr, &sum);
    if (tid < E) off[tid] = ex;
    if (tid == 0) off[E] = sum;
    __syncthreads();

    write_layout(o, off, total, E, B, S, C, tid, kAlignThreads);

    for (int e = tid; e < E; e += kAlignThreads)
        for (int v = 0; v < kAlignWaves; ++v) hist[v * E + e] += off[e];
    __syncthreads();
    walk_slots<true>(ids, s0, s1, E, nbits, hist + w * E, o.sorted);
}

// ---------------------------------------------------------------- 2 launches --
__global__ void __launch_bounds__(kAlignThreads)
align_count_kernel(const int32_t* __restrict__ ids, int64_t S, int E, int nbits, int64_t chunk,
                   int32_t* __restrict__ counts) {
    extern __shared__ int lds[];
    int* hist = lds;
    const int tid = threadIdx.x, w = tid / kWave, b = blockIdx.x;
    for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) hist[i] = 0;
    __syncthreads();
    const int64_t c0 = (int64_t)b * chunk;
    const int64_t c1 = c0 + chunk < S ? c0 + chunk : S;
    int64_t s0, s1;
    wave_range(c0 < S ? c0 : S, c1, w, &s0, &s1);
    walk_slots<false>(ids, s0, s1, E, nbits, hist + w * E, nullptr);
    __syncthreads();
    for (int e = tid; e < E; e += kAlignThreads) {
        int c = 0;
        for (int v = 0; v < kAlignWaves; ++v) c += hist[v * E + e];
        counts[(int64_t)b * E + e] = c;
    }
}

__global__ void __launch_bounds__(kAlignThreads)
align_place_kernel(const int32_t* __restrict__ ids, int64_t S, int E, int B, int nbits, int64_t C,
                   int64_t chunk, int G, int e_up, const int32_t* __restrict__ counts, AlignOut o) {
    extern __shared__ int lds[];
    int* hist = lds;                               // [waves][E]
    int* off = hist + kAlignWaves * E;             // [E+1]
    int* total = off + E + 1;                      // [E]
    int* scr = total + E;                          // [16]
    int* part = scr + 16;                          // [1024] partial sums, then bases
    int* part_all = part + kAlignThreads;          // [1024]
    const int tid = threadIdx.x, w = tid / kWave, b = blockIdx.x;

    // merge: per expert, the count before this workgroup and the total
    {
        const int e = tid % e_up, split = kAlignThreads / e_up, r = tid / e_up;
        int before = 0, all = 0;
        if (e < E) {
            for (int bb = r; bb < G; bb += split) {
                const int c = counts[(int64_t)bb * E + e];
                all += c;
                before += (bb < b) ? c : 0;
            }
        }
        part[tid] = before;
        part_all[tid] = all;
    }
    for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) hist[i] = 0;
    __syncthreads();
    int padded = 0, base_e = 0;
    if (tid < E) {
        const int split = kAlignThreads / e_up;
        int all = 0;
        for (int r = 0; r < split; ++r) {
            base_e += part[r * e_up + tid];
            all += part_all[r * e_up + tid];
        }
        total[tid] = all;
        padded = (all + B - 1) / B * B;
    }
    int sum;
    const int ex = block_excl_scan(tid < E ? padded : 0, scr, &sum);
    if (tid < E) off[tid] = ex;
    if (tid == 0) off[E] = sum;

    // recount this workgroup's chunk per wave
    const int64_t c0 = (int64_t)b * chunk;
    const int64_t c1 = c0 + chunk < S ? c0 + chunk : S;
    int64_t s0, s1;
    wave_range(c0 < S ? c0 : S, c1, w, &s0, &s1);
    walk_slots<false>(ids, s0, s1, E, nbits, hist + w * E, nullptr);
    __syncthreads();

    write_layout(o, off, total, E, B, S, C, (int64_t)b * kAlignThreads + tid,
                 (int64_t)G * kAlignThreads);

    if (tid < E) {
        int run = off[tid] + base_e;
        for (int v = 0; v < kAlignWaves; ++v) {
            const int c = hist[v * E + tid];
            hist[v * E + tid] = run;
            run += c;
        }
    }
    __syncthreads();
    walk_slots<true>(ids, s0, s1, E, nbits, hist + w * E, o.sorted);
}

// ------------------------------------------------------------------- host --
int align_nbits(int E) {
    int n = 0;
    while ((1 << n) < E) ++n;
    return n;
}

AlignPlan align_plan(int64_t S, int E) {
    AlignPlan p;
    p.single = S <= kAlignSingleMaxSlots;
    p.G = 0;
    p.chunk = 0;
    if (!p.single) {
        int64_t g = (S + kAlignSlotsPerWg - 1) / kAlignSlotsPerWg;
        g = (g + kNumXcd - 1) / kNumXcd * kNumXcd;
        if (g < kNumXcd) g = kNumXcd;
        if (g > kAlignMaxWg) g = kAlignMaxWg;
        int64_t chunk = (S + g - 1) / g;
        chunk = (chunk + kWave - 1) / kWave * kWave;
        p.G = (int)g;
        p.chunk = chunk;
    }
    p.workspace_bytes = p.single ? 0 : (int64_t)p.G * E * (int64_t)sizeof(int32_t);
    return p;
}

hipError_t launch_align_sort(const int32_t* ids, int64_t S, int E, int B, int64_t C,
                             int32_t* sorted, int32_t* expert_ids, int32_t* post_padded,
                             int32_t* offsets, void* workspace, hipStream_t stream) {
    const AlignPlan plan = align_plan(S, E);
    const int nbits = align_nbits(E);
    AlignOut o{sorted, expert_ids, post_padded, offsets};
    if (plan.single) {
        const size_t lds = align_lds_ints(E) * sizeof(int);
        hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(kAlignThreads), lds, stream, ids, S, E,
                           B, nbits, C, o);
        return hipGetLastError();
    }
    int32_t* counts = static_cast<int32_t*>(workspace);
    hipLaunchKernelGGL(align_count_kernel, dim3(plan.G), dim3(kAlignThreads),
                       (size_t)kAlignWaves * E * sizeof(int), stream, ids, S, E, nbits, plan.chunk,
                       counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    int e_up = kWave;
    while (e_up < E) e_up <<= 1;
    const size_t lds = (align_lds_ints(E) + 2 * kAlignThreads) * sizeof(int);
    hipLaunchKernelGGL(align_place_kernel, dim3(plan.G), dim3(kAlignThreads), lds, stream, ids, S, E,
                       B, nbits, C, plan.chunk, plan.G, e_up, (const int32_t*)counts, o);
    return hipGetLastError();
}

}  // namespace moe
