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
// * Each workgroup of 1024 threads owns a chunk of 1024*R consecutive slots
//   (R slots per thread, held in registers from coalesced reads).  Wave w owns
//   the contiguous sub-chunk [64*R*w, 64*R*(w+1)) and walks it in 64-slot
//   steps, so a slot's stable position inside its expert's run is: the run's
//   start in the chunk + the counts of earlier waves + the wave's count before
//   this step + the lanes of this step below it with the same expert.
// * That last term comes from a per-wave LDS bit-mask per expert: each lane
//   ORs its lane bit into its expert's mask (ds_or_b64; order does not matter)
//   and reads the mask back (the wave's LDS instructions run in order, so the
//   read sees the whole step); its rank is the popcount below its lane and
//   the lowest lane advances the wave's count and clears the mask.  A few LDS
//   operations per step instead of one ballot per id bit.  Where the masks do
//   not fit in LDS (more than ~600 experts) the ballots are used.
// * The chunk is then sorted by expert in LDS -- packed (expert << 16 |
//   local slot) words -- and every expert's run of it is written to its final
//   place with consecutive threads on consecutive addresses, so the scatter
//   into sorted_token_ids is coalesced instead of one 4-byte write per slot.
// * Up to 4096 slots: ONE workgroup.  Larger: G workgroups, G a multiple of
//   the 8 XCDs, in ONE launch when all of them can be resident at once: each
//   publishes its chunk's counts, a grid barrier (counter in the workspace,
//   bounded wait) orders them, and each workgroup merges the small count
//   matrix itself; with a larger matrix the workgroups first scan its
//   columns (one expert per wave) and meet at a second barrier.  With at
//   most 16 workgroups there is no barrier: the counts are published as
//   words tagged with the call's generation, and each workgroup loads the
//   matrix again (bounded) until every tag is this call's.  Larger
//   still, the counts come from a count launch (+ a scan launch) and the
//   place launch does the rest.  Padding, the tail and expert_ids are written
//   by all workgroups in a grid-strided pattern.
// * Cross-XCD ordering at a barrier: the shared counts are written and read
//   with agent-scope accesses (they bypass the per-XCD L2); every wave waits
//   for its stores, then one thread bumps the counter and polls it.  The
//   last workgroup past the final barrier resets the counters, so the
//   workspace is left as it was found (zero).
// * Barriers inside a workgroup order LDS only, so global loads and stores
//   in flight are not drained at each one.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr unsigned kAlignWaitVmem = 0xF70;       // s_waitcnt vmcnt(0)
constexpr int kAlignSpinLimit = 1 << 22;         // polls of a barrier before it gives up
// Barrier words at the head of the workspace, each counter on its own
// 128-byte line: [0] status, [32] top-level arrivals, [64 + 32 g] arrivals of
// group g, [576 + 32 g] release generation of group g (g < 16; a group is 16
// consecutive workgroups).  Counters are zero between calls; generations may
// hold anything.
constexpr int kAlignGroup = 16;
constexpr int kAlignMaxGroups = 16;
constexpr int kAlignLine = 32;
constexpr int kAlignCtlInts = 2 * kAlignLine + 2 * kAlignMaxGroups * kAlignLine;   // 1088

struct AlignCtl {
    int* status;       // sticky: nonzero once a wait gave up
    int* top;          // groups whose workgroups all arrived (this phase)
    int* group;        // [g * kAlignLine] workgroups of group g that arrived (this phase)
    int* gen;          // [g * kAlignLine] bumped once per completed barrier
};

// A workgroup barrier that orders LDS only: it waits for the wave's LDS
// operations, not for its global loads and stores in flight (which
// __syncthreads() also waits for), so id loads keep streaming and output
// stores keep draining across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Device-wide data shared across XCDs (counts, bases, totals) is written and
// read with agent-scope atomic accesses, which bypass the per-XCD L2, so a
// barrier needs no L2 write-back or invalidate (32 workgroups per XCD each
// writing back and invalidating the L2 cost ~10 us per barrier).
__device__ __forceinline__ int load_shared(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_shared(int32_t* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_shared64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_shared64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// With few workgroups the merge needs no barrier: every count is published
// as a 64-bit word (tag << 32 | count) and read back until its tag is this
// call's.  The tag has its top bit set (plain counts and totals that the
// other paths write into the same workspace never do) and comes from the
// generation word of group 0 read at the kernel's start, + 1; every
// workgroup stores that value back at its end.  No workgroup can end before
// all have published, and publishing needs the generation already read, so
// every workgroup reads the same value; a word left by an earlier call holds
// an older tag.
__device__ __forceinline__ uint32_t merge_tag(int gen) {
    return 0x80000000u | ((uint32_t)(gen + 1) & 0x7FFFFFFFu);
}

enum AlignMode : int {
    kSingle = 0,       // one workgroup: no counts to merge
    kFused = 1,        // counts, grid barrier(s) and placement in one launch
    kPlace = 2,        // counts (or bases) from earlier launches
    kTagged = 3,       // one launch, few workgroups: tagged counts, no barrier
};

// Exclusive prefix sums of two values over the 1024 threads of a workgroup
// at once; *tot_a / *tot_b get the sums.  lds32 is 32 ints of scratch.
__device__ __forceinline__ void block_excl_scan2(int a, int b, int* lds32, int* ex_a, int* ex_b, int* tot_a,
                                                 int* tot_b) {
    const int w = threadIdx.x / kWave;
    const int ia = wave_incl_scan_i32(a), ib = wave_incl_scan_i32(b);
    if (lane_id() == kWave - 1) {
        lds32[w] = ia;
        lds32[kAlignWaves + w] = ib;
    }
    lds_barrier();
    int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < kAlignWaves; ++i) {
        const int ta = lds32[i], tb = lds32[kAlignWaves + i];
        ba += (i < w) ? ta : 0;
        bb += (i < w) ? tb : 0;
        sa += ta;
        sb += tb;
    }
    lds_barrier();
    *ex_a = ba + ia - a;
    *ex_b = bb + ib - b;
    *tot_a = sa;
    *tot_b = sb;
}

struct AlignOut {
    int32_t* sorted;
    int32_t* expert_ids;
    int32_t* post_padded;
    int32_t* offsets;
};

struct AlignArgs {
    const int32_t* ids;
    int64_t S, C;
    int E, B, log2B, G;
    int merge;         // G > 1: each workgroup merges the [G,E] counts itself (else column scans)
    int32_t* counts;   // [G,E] workgroup-major (merge) or [E,G] expert-major (scan)
    int32_t* totals;   // [E] (scan)
    int* ctl;          // kFused: the barrier words
    AlignOut o;
};

// x / B; log2B >= 0 when B is a power of two (a shift instead of a division)
__device__ __forceinline__ int div_block(int x, int B, int log2B) { return log2B >= 0 ? x >> log2B : x / B; }

// Writes everything that depends only on the aligned offsets: P, offsets,
// expert_ids, the padding inside every expert's run and the tail [P, C).
// gthread/gstride index the threads of the whole grid (waves whole): each
// expert's padding and block ids are written by one wave with consecutive
// lanes on consecutive addresses; the tail is spread over all threads.
__device__ void write_layout(const AlignOut& o, const int* off, const int* total, int E, int B, int log2B,
                             int64_t S, int64_t C, int64_t gthread, int64_t gstride) {
    // positions fit in int32 (S + C < 2^31 is a precondition)
    const int P = off[E], Ci = (int)C, sent = (int)S;
    const int gt = (int)gthread, gs = (int)gstride;
    if (gt == 0) o.post_padded[0] = P;
    if (o.offsets)
        for (int e = gt; e <= E; e += gs) o.offsets[e] = off[e];
    // wave gw takes experts gw, gw + nw, ...: lane k first reads the offsets
    // of the k-th of a group of 64 of them (one LDS round trip), then the wave
    // walks the group with the values broadcast from lane k
    const int lane = gt & (kWave - 1), gw = gt / kWave, nw = gs / kWave;
    for (int e0 = gw; e0 < E; e0 += kWave * nw) {
        const int mine = e0 + lane * nw;
        int o0 = 0, o1 = 0, t = 0;
        if (mine < E) {
            o0 = off[mine];
            o1 = off[mine + 1];
            t = total[mine];
        }
        const int nk = (E - e0 + nw - 1) / nw < kWave ? (E - e0 + nw - 1) / nw : kWave;
        for (int k = 0; k < nk; ++k) {
            const int a0 = __builtin_amdgcn_readlane(o0, k), a1 = __builtin_amdgcn_readlane(o1, k);
            const int at = __builtin_amdgcn_readlane(t, k);
            for (int p = a0 + at + lane; p < a1; p += kWave) o.sorted[p] = sent;
            const int j1 = div_block(a1, B, log2B);
            for (int j = div_block(a0, B, log2B) + lane; j < j1; j += kWave) o.expert_ids[j] = e0 + k * nw;
        }
    }
    for (int p = P + gt; p < Ci; p += gs) o.sorted[p] = sent;
    const int jt = div_block(Ci, B, log2B);
    for (int j = div_block(P, B, log2B) + gt; j < jt; j += gs) o.expert_ids[j] = -1;
}

// LDS ints of the kernel: per-wave counts [16][E]; per expert the chunk count
// / local offset, the aligned offset, the total and the output offset
// [4][E+1]; scan scratch [32]; then one region that holds the per-wave
// expert masks [16][E] (u64) while ranking and the sorted chunk [1024*R]
// afterwards.
__host__ __device__ inline int64_t align_region_ints(int E, int R, bool masks) {
    const int64_t region = (int64_t)kAlignThreads * R;
    const int64_t mask_ints = masks ? 2 * (int64_t)kAlignWaves * E : 0;
    return region > mask_ints ? region : mask_ints;
}
__host__ __device__ inline int64_t align_lds_ints(int E, int R, bool masks) {
    return (int64_t)kAlignWaves * E + 4 * (int64_t)(E + 1) + 32 + align_region_ints(E, R, masks);
}
constexpr int64_t kAlignLdsInts = 40000;        // 160 000 bytes of the 160 KiB
constexpr int kAlignMaxR = 32;
constexpr int kAlignSingleMax = 4096;           // slots handled by one workgroup
constexpr int kAlignMaxWg = 256;                // grow the chunk rather than the grid beyond this
constexpr int64_t kAlignMergeMaxInts = 16384;   // a [G,E] matrix up to this is merged by every workgroup
// Up to this many workgroups the merge uses tagged count words instead of a
// grid barrier: measured at 1024 tokens x 8 (8 workgroups) 7.3 against
// 8.6 us; at 16384 x 8 (64 workgroups, more polling) 10.8 against 9.9.
#ifndef MOE_ALIGN_TAGGED_MAX_WG
#define MOE_ALIGN_TAGGED_MAX_WG 16
#endif
constexpr int kAlignTaggedMaxWg = MOE_ALIGN_TAGGED_MAX_WG;
// Slots per thread of the multi-workgroup path (grown beyond 256 workgroups).
#ifndef MOE_ALIGN_MIN_R
#define MOE_ALIGN_MIN_R 2
#endif

// ------------------------------------------------------------ stable ranks --
// ev[j] (an expert id, or -1) becomes e | p << 16, p the position of slot j
// among the wave's slots of expert e in ascending slot order (p < 64*R); one
// register per slot.  run_w[e] ends as the wave's count of e.

// Per-step masks in LDS: the lanes of a step that hold expert e each OR their
// bit into e's 64-lane mask (one dword each: lanes 0-31 into its low half,
// 32-63 into its high half); reading the mask back gives the lanes below
// with the same e (the wave's LDS operations complete in order, so the read
// sees every OR of the step).  The rank adds the wave's count of e so far,
// and the lowest lane advances that count and clears the mask.  8-byte masks
// and 4-byte counts in separate arrays: measured faster than 16-byte records
// holding both, or four 16-lane masks per expert (fewer same-address
// collisions, more bytes and bank conflicts).
template <int R>
__device__ __forceinline__ void rank_by_masks(int (&ev)[R], int* run_w, uint64_t* mask_w, int lane) {
    const uint32_t bit = 1u << (lane & 31);
    uint32_t* half = reinterpret_cast<uint32_t*>(mask_w) + (lane >> 5);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int e = ev[j];
        if (e >= 0) {
            __hip_atomic_fetch_or(half + 2 * e, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            const uint64_t m = __hip_atomic_load(mask_w + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            const int r = popc_below(m);
            const int pos = __hip_atomic_load(run_w + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            ev[j] = e | (pos + r) << 16;
            if (r == 0) {                         // the lowest lane of the group
                __hip_atomic_store(run_w + e, pos + (int)__popcll(m), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_store(mask_w + e, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
}

// Ballots (any E up to 2^NB): the mask of lanes with the same id is the AND
// over the NB id bits of the ballot of that bit or its complement.
template <int R, int NB>
__device__ __forceinline__ void rank_by_ballots(int (&ev)[R], int* run_w) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const bool valid = ev[j] >= 0;
        const int e = valid ? ev[j] : 0;
        const uint64_t v = ballot(valid);
        uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t s = 0u - (uint32_t)((e >> b) & 1);      // all ones where the bit is set
            const uint64_t m = ballot(s != 0);
            lo &= ~(s ^ (uint32_t)m);
            hi &= ~(s ^ (uint32_t)(m >> 32));
        }
        if (valid) {
            const int r = (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
            const int pos = __hip_atomic_load(run_w + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            ev[j] = e | (pos + r) << 16;
            if (r == 0)
                __hip_atomic_store(run_w + e, pos + __popc(lo) + __popc(hi), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
}

// -------------------------------------------------------------- grid barrier --
// Same-address device atomics serialize at about 40 ns each, so the G
// workgroups arrive in two levels: each adds to its group's counter (16 per
// line), the last of a group adds to the top counter, and the last group's
// last workgroup bumps every group's generation, which the waiters poll (16
// per line).  Counters accumulate over the phases of a call (phase k waits
// for k times the members), and the releaser of the last phase clears them
// after releasing, for the next call.  A waiter compares the generation with
// the value it read at the kernel's start, so generations need no reset.
// Before arriving, every wave waits for its own stores (the shared data,
// written with agent-scope stores, is then at the coherence point).
// Bounded: past kAlignSpinLimit polls the status word is set and the
// workgroup goes on (the result is then wrong, and the status says so).
__device__ __forceinline__ AlignCtl align_ctl(int* w) {
    return AlignCtl{w, w + kAlignLine, w + 2 * kAlignLine, w + 2 * kAlignLine + kAlignMaxGroups * kAlignLine};
}

__device__ __forceinline__ int atomic_add_agent(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// phase k of `phases` (1-based); gen0 = this group's generation at the
// kernel's start (thread 0's value)
__device__ __forceinline__ void grid_barrier(const AlignCtl& c, int G, int k, int phases, int gen0) {
    __builtin_amdgcn_s_waitcnt(kAlignWaitVmem);
    lds_barrier();
    if (threadIdx.x == 0) {
        const int g = blockIdx.x / kAlignGroup, ng = (G + kAlignGroup - 1) / kAlignGroup;
        const int members = G - g * kAlignGroup < kAlignGroup ? G - g * kAlignGroup : kAlignGroup;
        if (atomic_add_agent(c.group + g * kAlignLine, 1) == k * members - 1 &&
            atomic_add_agent(c.top, 1) == k * ng - 1) {
            // everyone has arrived: release every group; after the last
            // phase nobody reads the counters again in this call
            for (int i = 0; i < ng; ++i) atomic_add_agent(c.gen + i * kAlignLine, 1);
            if (k == phases) {
                for (int i = 0; i < ng; ++i) store_shared(c.group + i * kAlignLine, 0);
                store_shared(c.top, 0);
            }
        }
        int polls = 0;
        while (load_shared(c.gen + g * kAlignLine) - gen0 < k) {
            if (++polls > kAlignSpinLimit) {
                __hip_atomic_fetch_or(c.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    lds_barrier();
}

// One expert's row of the expert-major [E,G] counts, by one wave: the
// exclusive prefix over workgroups, in place, and the expert's total.  Lane l
// owns a contiguous run of the row.  PER > 0: at most PER entries per lane
// (G <= 64 * PER), loaded all at once, so the row costs one memory round
// trip for the loads and one for the stores; PER == 0: any G, serially.
template <int PER>
__device__ __forceinline__ void scan_expert_row(int32_t* __restrict__ counts, int G, int e,
                                                int32_t* __restrict__ totals) {
    const int lane = lane_id();
    int32_t* row = counts + (int64_t)e * G;
    const int per = (G + kWave - 1) / kWave;
    const int b0 = lane * per < G ? lane * per : G;
    const int b1 = b0 + per < G ? b0 + per : G;
    if constexpr (PER > 0) {
        int c[PER];
        int sum = 0;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            c[u] = b0 + u < b1 ? load_shared(row + b0 + u) : 0;
            sum += c[u];
        }
        const int incl = wave_incl_scan_i32(sum);
        int run = incl - sum;
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (b0 + u < b1) {
                store_shared(row + b0 + u, run);
                run += c[u];
            }
        if (lane == kWave - 1) store_shared(totals + e, incl);
    } else {
        int sum = 0;
        for (int b = b0; b < b1; ++b) sum += load_shared(row + b);
        const int incl = wave_incl_scan_i32(sum);
        int run = incl - sum;
        for (int b = b0; b < b1; ++b) {
            const int c = load_shared(row + b);
            store_shared(row + b, run);
            run += c;
        }
        if (lane == kWave - 1) store_shared(totals + e, incl);
    }
}

// ------------------------------------------------------------------- count --
// (kPlace path) Counts of each expert in each workgroup's chunk:
// workgroup-major (counts[b * E + e], merged by the place workgroups) or, for
// the scan launch, expert-major (counts[e * G + b]).  The order of the slots
// does not matter here, so a thread reads 4 consecutive ids at a time and adds
// with LDS atomics.
template <int R>
__global__ void __launch_bounds__(kAlignThreads)
align_count_kernel(const int32_t* __restrict__ ids, int64_t S, int E, int G, int expert_major,
                   int32_t* __restrict__ counts) {
    extern __shared__ int lds[];
    int* hist = lds;                               // [E]
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kAlignThreads) hist[e] = 0;
    const int64_t c0 = (int64_t)blockIdx.x * (kAlignThreads * R);
    constexpr int kQuads = (R + 3) / 4;            // 4-id groups per thread
    const bool vec = (reinterpret_cast<uintptr_t>(ids) & 15) == 0;
    int ev[4 * kQuads];
#pragma unroll
    for (int q = 0; q < kQuads; ++q) {
        const int64_t i = c0 + 4 * ((int64_t)q * kAlignThreads + tid);
        if (vec && i + 3 < S && 4 * (q * kAlignThreads + tid) + 3 < kAlignThreads * R) {
            const int4 v = *reinterpret_cast<const int4*>(ids + i);
            ev[4 * q] = v.x; ev[4 * q + 1] = v.y; ev[4 * q + 2] = v.z; ev[4 * q + 3] = v.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool in = i + u < S && 4 * (q * kAlignThreads + tid) + u < kAlignThreads * R;
                ev[4 * q + u] = in ? ids[i + u] : -1;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4 * kQuads; ++j)
        if (ev[j] >= 0 && ev[j] < E) atomicAdd(&hist[ev[j]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += kAlignThreads)
        counts[expert_major ? (int64_t)e * G + blockIdx.x : (int64_t)blockIdx.x * E + e] = hist[e];
}

// (kPlace path) Per expert, one wave each: the row scan of the expert-major counts.
__global__ void __launch_bounds__(kAlignThreads)
align_scan_kernel(int32_t* __restrict__ counts, int G, int E, int32_t* __restrict__ totals) {
    const int e = blockIdx.x * kAlignWaves + threadIdx.x / kWave;
    if (e >= E) return;                            // whole waves
    scan_expert_row<0>(counts, G, e, totals);
}

// ------------------------------------------------------------------ kernel --
// RANK: 0 = per-wave LDS masks, else ballots over RANK id bits.
template <int R, int MODE, int RANK>
__global__ void __launch_bounds__(kAlignThreads) align_kernel(AlignArgs a) {
    extern __shared__ int lds[];
    const int E = a.E, G = a.G;
    int* run = lds;                                // [waves][E] counts, then bases
    int* loc = run + kAlignWaves * E;              // [E+1] chunk counts, then local offsets
    int* off = loc + (E + 1);                      // [E+1] aligned offsets
    int* tot = off + (E + 1);                      // [E+1] expert totals
    int* gof = tot + (E + 1);                      // [E+1] output offset of local position 0
    int* scr = gof + (E + 1);                      // [32]
    uint32_t* chunk = reinterpret_cast<uint32_t*>(scr + 32);   // [1024*R] after ranking
    uint64_t* masks = reinterpret_cast<uint64_t*>(scr + 32);   // [waves][E] while ranking
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id(), b = blockIdx.x;

    AlignCtl ctl{};
    int gen0 = 0;      // thread 0: its group's barrier generation (tagged: group 0's)
    if (MODE == kFused || MODE == kTagged) {
        ctl = align_ctl(a.ctl);
        if (tid == 0) gen0 = load_shared(ctl.gen + (MODE == kTagged ? 0 : (b / kAlignGroup) * kAlignLine));
    }
    for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) {
        run[i] = 0;
        if (RANK == 0) masks[i] = 0;
    }
    lds_barrier();

    // this thread's slots: wave w's sub-chunk, one 64-slot step per j (the
    // loads are issued after the barrier, so step j waits only for its own)
    const int64_t c0 = (int64_t)b * (kAlignThreads * R);
    const int wfirst = w * (kWave * R) + lane;     // local index of this thread's first slot
    int ev[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t i = c0 + wfirst + j * kWave;
        const int e = i < a.S ? a.ids[i] : -1;
        ev[j] = (e >= 0 && e < E) ? e : -1;        // ids outside [0,E) are skipped
    }

    if constexpr (RANK == 0)
        rank_by_masks<R>(ev, run + w * E, masks + w * E, lane);
    else
        rank_by_ballots<R, RANK>(ev, run + w * E);
    // the tag, for every thread (off[] is not in use yet; the generation
    // load has long returned)
    if (MODE == kTagged && tid == 0) off[E] = gen0;
    lds_barrier();

    // per expert: wave bases (exclusive over waves) and the chunk count
    int mine = 0;
    if (tid < E) {
        int c[kAlignWaves];
#pragma unroll
        for (int v = 0; v < kAlignWaves; ++v) c[v] = run[v * E + tid];
#pragma unroll
        for (int v = 0; v < kAlignWaves; ++v) {
            run[v * E + tid] = mine;
            mine += c[v];
        }
    }

    // this workgroup's base in each expert and the expert totals
    int base_e = 0, all_e = mine;
    const uint32_t tag = MODE == kTagged ? merge_tag(off[E]) : 0u;
    uint64_t* const counts64 = reinterpret_cast<uint64_t*>(a.counts);
    if (MODE == kTagged && tid < E)
        store_shared64(counts64 + (int64_t)b * E + tid, ((uint64_t)tag << 32) | (uint32_t)mine);
    if (MODE == kFused) {
        if (tid < E) store_shared(a.counts + (a.merge ? (int64_t)b * E + tid : (int64_t)tid * G + b), mine);
        const int phases = a.merge ? 1 : 2;
        grid_barrier(ctl, G, 1, phases, gen0);
        if (!a.merge) {
            // the columns of the expert-major matrix: one expert per wave
            for (int e = b * kAlignWaves + w; e < E; e += G * kAlignWaves)
                scan_expert_row<kAlignGroup * kAlignMaxGroups / kWave>(a.counts, G, e, a.totals);
            grid_barrier(ctl, G, 2, phases, gen0);
        }
    }
    if (MODE != kSingle) {
        if (!a.merge) {
            if (tid < E) {
                base_e = load_shared(a.counts + (int64_t)tid * G + b);
                all_e = load_shared(a.totals + tid);
            }
        } else {
            // every entry of the small [G,E] matrix is loaded in one memory
            // round trip: thread (part, e) sums rows part, part + parts, ... of
            // column e (e fastest across lanes, so each row is read coalesced;
            // e_up and parts are powers of two)
            int e_up = kWave;
            while (e_up < E) e_up <<= 1;
            const int parts = kAlignThreads / e_up, e = tid & (e_up - 1), part = tid / e_up;
            constexpr int kBatch = 16;
            int before = 0, all = 0;
            if (e < E) {
                for (int bb0 = part; bb0 < G; bb0 += kBatch * parts) {
                    int c[kBatch];
                    if (MODE == kTagged) {
                        // all loaded at once, and all loaded again while any
                        // is not yet published in this call (or until the
                        // wait gives up)
                        uint64_t t[kBatch];
                        for (int polls = 0;; ++polls) {
#pragma unroll
                            for (int u = 0; u < kBatch; ++u) {
                                const int bb = bb0 + u * parts;
                                t[u] = bb < G ? load_shared64(counts64 + (int64_t)bb * E + e) : (uint64_t)tag << 32;
                            }
                            bool ready = true;
#pragma unroll
                            for (int u = 0; u < kBatch; ++u) ready &= (uint32_t)(t[u] >> 32) == tag;
                            if (ready) break;
                            if (polls == kAlignSpinLimit) {
                                __hip_atomic_fetch_or(ctl.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                break;
                            }
                            __builtin_amdgcn_s_sleep(2);
                        }
#pragma unroll
                        for (int u = 0; u < kBatch; ++u) c[u] = (int)(uint32_t)t[u];
                    } else {
#pragma unroll
                        for (int u = 0; u < kBatch; ++u) {
                            const int bb = bb0 + u * parts;
                            c[u] = bb < G ? load_shared(a.counts + (int64_t)bb * E + e) : 0;
                        }
                    }
#pragma unroll
                    for (int u = 0; u < kBatch; ++u) {
                        all += c[u];
                        before += bb0 + u * parts < b ? c[u] : 0;
                    }
                }
            }
            int* pb = reinterpret_cast<int*>(chunk);   // scratch: the chunk is not in use yet
            pb[tid] = before;
            pb[kAlignThreads + tid] = all;
            lds_barrier();
            all_e = 0;
            if (tid < E)
                for (int r = 0; r < parts; ++r) {
                    base_e += pb[r * e_up + tid];
                    all_e += pb[kAlignThreads + r * e_up + tid];
                }
        }
    }
    int nvalid, ptotal, lo, ex;
    block_excl_scan2(tid < E ? mine : 0, tid < E ? (all_e + a.B - 1) / a.B * a.B : 0, scr, &lo, &ex, &nvalid,
                     &ptotal);
    if (tid < E) {
        loc[tid] = lo;
        off[tid] = ex;
        tot[tid] = all_e;
        gof[tid] = ex + base_e - lo;
#pragma unroll
        for (int v = 0; v < kAlignWaves; ++v) run[v * E + tid] += lo;   // wave base inside the sorted chunk
    }
    if (tid == 0) off[E] = ptotal;
    lds_barrier();

    write_layout(a.o, off, tot, E, a.B, a.log2B, a.S, a.C, (int64_t)b * kAlignThreads + tid,
                 (int64_t)G * kAlignThreads);

    // every slot to its stable position inside the sorted chunk
#pragma unroll
    for (int j = 0; j < R; ++j)
        if (ev[j] >= 0) {
            const int e = ev[j] & 0xFFFF, p = ev[j] >> 16;
            chunk[run[w * E + e] + p] = ((uint32_t)e << 16) | (uint32_t)(wfirst + j * kWave);
        }
    lds_barrier();

    // coalesced write-out: position idx of the sorted chunk is slot c0 + local
    for (int idx = tid; idx < nvalid; idx += kAlignThreads) {
        const uint32_t v = chunk[idx];
        a.o.sorted[gof[v >> 16] + idx] = (int32_t)(c0 + (v & 0xFFFFu));
    }
    // the generation moves on for the next call (the same value from every
    // workgroup)
    if (MODE == kTagged && tid == 0) store_shared(ctl.gen, gen0 + 1);
}

// ------------------------------------------------------------------- host --
static bool align_masks_fit(int E, int R) { return align_lds_ints(E, R, true) <= kAlignLdsInts; }

static int align_max_r(int E) {
    // the largest chunk that fits with the masks, or else with the ballots
    int r = kAlignMaxR;
    while (r > 1 && align_lds_ints(E, r, false) > kAlignLdsInts) r >>= 1;
    return r;
}

AlignPlan align_plan(int64_t S, int E) {
    AlignPlan p;
    const int rmax = align_max_r(E);
    int r = 1;
    if (S <= kAlignSingleMax) {
        while ((int64_t)kAlignThreads * r < S) r <<= 1;
        p.G = 1;
    } else {
        // two slots per thread, or one when eight one-slot chunks cover S
        r = S <= (int64_t)kNumXcd * kAlignThreads ? 1 : MOE_ALIGN_MIN_R;
        while (r < rmax && (S + (int64_t)kAlignThreads * r - 1) / ((int64_t)kAlignThreads * r) > kAlignMaxWg) r <<= 1;
        const int64_t g = (S + (int64_t)kAlignThreads * r - 1) / ((int64_t)kAlignThreads * r);
        p.G = (int)((g + kNumXcd - 1) / kNumXcd * kNumXcd);    // whole rounds of the 8 XCDs
    }
    p.R = r;
    p.single = p.G == 1;
    p.masks = align_masks_fit(E, r);
    // the in-kernel merge borrows 2048 ints of the chunk region
    p.merge = (int64_t)p.G * E <= kAlignMergeMaxInts && align_region_ints(E, r, p.masks) >= 2 * kAlignThreads;
    p.tagged = p.merge && p.G <= kAlignTaggedMaxWg;
    p.chunk = (int64_t)kAlignThreads * r;
    p.workspace_bytes =
        p.single ? 0
                 : ((int64_t)kAlignCtlInts + (int64_t)p.G * E * (p.tagged ? 2 : 1) + (p.merge ? 0 : E)) *
                       (int64_t)sizeof(int32_t);
    return p;
}

// One-time per-device set-up, race-free: hipFuncSetAttribute applies to the
// current device, so each device gets its own once-flag.
constexpr int kMaxDevices = 64;

static hipError_t current_device(int* dev) {
    hipError_t err = hipGetDevice(dev);
    if (err != hipSuccess) return err;
    return (*dev < 0 || *dev >= kMaxDevices) ? hipErrorInvalidDevice : hipSuccess;
}

// The dynamic-LDS limit of one kernel instantiation, raised once per device.
template <int R, int MODE, int RANK>
static hipError_t lds_opt_in() {
    static std::once_flag once[kMaxDevices];
    static hipError_t result[kMaxDevices];
    int dev = 0;
    hipError_t err = current_device(&dev);
    if (err != hipSuccess) return err;
    std::call_once(once[dev], [dev] {
        result[dev] = hipFuncSetAttribute((const void*)align_kernel<R, MODE, RANK>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)(kAlignLdsInts * sizeof(int)));
    });
    return result[dev];
}

// Compute units of the current device (workgroups of the single-launch path
// that are surely resident together: one per CU).
static hipError_t device_cus(int* cus) {
    static std::once_flag once[kMaxDevices];
    static int n[kMaxDevices];
    static hipError_t result[kMaxDevices];
    int dev = 0;
    hipError_t err = current_device(&dev);
    if (err != hipSuccess) return err;
    std::call_once(once[dev], [dev] {
        result[dev] = hipDeviceGetAttribute(&n[dev], hipDeviceAttributeMultiprocessorCount, dev);
    });
    *cus = n[dev];
    return result[dev];
}

template <int R, int MODE, int RANK>
static hipError_t launch_kernel(const AlignArgs& a, size_t lds, hipStream_t stream) {
    hipError_t err = lds_opt_in<R, MODE, RANK>();
    if (err != hipSuccess) return err;
    auto kern = align_kernel<R, MODE, RANK>;
    hipLaunchKernelGGL(kern, dim3(a.G), dim3(kAlignThreads), lds, stream, a);
    return hipGetLastError();
}

template <int R, int RANK>
static hipError_t launch_align_r(const AlignPlan& plan, AlignArgs a, void* workspace, hipStream_t stream) {
    const int E = a.E;
    const size_t lds = (size_t)align_lds_ints(E, R, RANK == 0) * sizeof(int);
    if (plan.single) return launch_kernel<R, kSingle, RANK>(a, lds, stream);
    a.ctl = static_cast<int*>(workspace);
    a.counts = static_cast<int32_t*>(workspace) + kAlignCtlInts;
    a.totals = plan.merge ? nullptr : a.counts + (int64_t)plan.G * E;
    int cus = 0;
    hipError_t err = device_cus(&cus);
    if (err != hipSuccess) return err;
    if (plan.tagged && plan.G <= cus) return launch_kernel<R, kTagged, RANK>(a, lds, stream);
    if (plan.G <= cus && plan.G <= kAlignGroup * kAlignMaxGroups)
        return launch_kernel<R, kFused, RANK>(a, lds, stream);
    // more workgroups than can surely be resident: count (+ scan) launches first
    hipLaunchKernelGGL(align_count_kernel<R>, dim3(plan.G), dim3(kAlignThreads), (size_t)E * sizeof(int), stream,
                       a.ids, a.S, E, plan.G, plan.merge ? 0 : 1, a.counts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (!plan.merge) {
        hipLaunchKernelGGL(align_scan_kernel, dim3((E + kAlignWaves - 1) / kAlignWaves), dim3(kAlignThreads), 0,
                           stream, a.counts, plan.G, E, a.totals);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return launch_kernel<R, kPlace, RANK>(a, lds, stream);
}

template <int R>
static hipError_t launch_align_rm(const AlignPlan& plan, const AlignArgs& a, void* workspace, hipStream_t stream) {
    if (plan.masks) return launch_align_r<R, 0>(plan, a, workspace, stream);
    return a.E <= 256 ? launch_align_r<R, 8>(plan, a, workspace, stream)
                      : launch_align_r<R, 10>(plan, a, workspace, stream);
}

// The no-allocation entry point's scratch: a fixed device array in place of
// the caller's workspace.  Every device holds its own copy at its own
// address; host code uses the address returned by hipGetSymbolAddress, never
// the array's name (which is a host-side stand-in).  Zero at load, and every
// call leaves its barrier words zero again.
static __device__ __align__(256) int32_t scratch[kAlignScratchBytes / sizeof(int32_t)];

hipError_t align_scratch_address(void** ptr) {
    static std::once_flag once[kMaxDevices];
    static void* addr[kMaxDevices];
    static hipError_t result[kMaxDevices];
    int dev = 0;
    hipError_t err = current_device(&dev);
    if (err != hipSuccess) return err;
    std::call_once(once[dev], [dev] { result[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch)); });
    if (result[dev] != hipSuccess) return result[dev];
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_align_sort(const int32_t* ids, int64_t S, int E, int B, int64_t C,
                             int32_t* sorted, int32_t* expert_ids, int32_t* post_padded,
                             int32_t* offsets, void* workspace, hipStream_t stream) {
    const AlignPlan plan = align_plan(S, E);
    AlignArgs a{};
    a.ids = ids;
    a.S = S;
    a.C = C;
    a.E = E;
    a.B = B;
    a.log2B = -1;
    if ((B & (B - 1)) == 0) {
        a.log2B = 0;
        while ((1 << a.log2B) < B) ++a.log2B;
    }
    a.G = plan.G;
    a.merge = plan.merge ? 1 : 0;
    a.o = AlignOut{sorted, expert_ids, post_padded, offsets};
    switch (plan.R) {
        case 1: return launch_align_rm<1>(plan, a, workspace, stream);
        case 2: return launch_align_rm<2>(plan, a, workspace, stream);
        case 4: return launch_align_rm<4>(plan, a, workspace, stream);
        case 8: return launch_align_rm<8>(plan, a, workspace, stream);
        case 16: return launch_align_rm<16>(plan, a, workspace, stream);
        case 32: return launch_align_rm<32>(plan, a, workspace, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
