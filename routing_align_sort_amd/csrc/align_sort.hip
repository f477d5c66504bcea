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
// * Stable ranks come from wave ballots, not atomics: for each 64-slot step a
//   wave builds, per lane, the mask of lanes holding the same expert from one
//   ballot per id bit; the lane's rank is the popcount of that mask below it
//   and the lowest lane advances the wave's running LDS counter.  Waves own
//   contiguous sub-chunks of their workgroup's chunk, so per-wave bases plus
//   running counts order every slot exactly as a stable sort does.
// * Each workgroup of 1024 threads owns a chunk of 1024*R consecutive slots
//   (R slots per thread, held in registers from one coalesced read).  It
//   sorts the chunk by expert in LDS -- packed (expert << 16 | local slot)
//   words -- and then writes every expert's run of the chunk to its final
//   place with consecutive threads on consecutive addresses, so the scatter
//   into sorted_token_ids is coalesced instead of one 4-byte write per slot.
// * Up to 4096 slots: ONE workgroup, one launch.  Larger: a count launch
//   (LDS atomics; order does not matter there) writes a [G,E] matrix to the
//   workspace, then the place launch.  Up to 64 workgroups every place
//   workgroup merges the small matrix itself (its base in each expert and the
//   expert totals: one L2 read instead of a grid-wide barrier across dies);
//   beyond that a scan launch turns the matrix into per-workgroup bases and
//   totals first.  Padding, the tail and expert_ids are written by all
//   workgroups in a grid-strided pattern.
#include <mutex>

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
    __syncthreads();
    int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < kAlignWaves; ++i) {
        const int ta = lds32[i], tb = lds32[kAlignWaves + i];
        ba += (i < w) ? ta : 0;
        bb += (i < w) ? tb : 0;
        sa += ta;
        sb += tb;
    }
    __syncthreads();
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

// Writes everything that depends only on the aligned offsets: P, offsets,
// expert_ids, the padding inside every expert's run and the tail [P, C).
// gthread/gstride index the threads of the whole grid (waves whole): each
// expert's padding and block ids are written by one wave with consecutive
// lanes on consecutive addresses; the tail is spread over all threads.
// x / B; log2B >= 0 when B is a power of two (a shift instead of a division)
__device__ __forceinline__ int div_block(int x, int B, int log2B) { return log2B >= 0 ? x >> log2B : x / B; }

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

// LDS ints of the place kernel: per-wave running counts [16][E]; per expert
// the chunk count / local offset, the aligned offset, the total and the
// output offset [4][E+1]; scan scratch [32]; the sorted chunk [1024*R].
__host__ __device__ inline int64_t align_place_lds_ints(int E, int R) {
    return (int64_t)kAlignWaves * E + 4 * (int64_t)(E + 1) + 32 + (int64_t)kAlignThreads * R;
}
constexpr int64_t kAlignLdsInts = 40000;        // 160 000 bytes of the 160 KiB
constexpr int kAlignMaxR = 32;
#ifndef MOE_ALIGN_MAX_WG
#define MOE_ALIGN_MAX_WG 256             // grow the chunk rather than the grid beyond this
#endif
#ifndef MOE_ALIGN_MIN_R
#define MOE_ALIGN_MIN_R 2
#endif
#ifndef MOE_ALIGN_MERGE_MAX_WG
#define MOE_ALIGN_MERGE_MAX_WG 64
#endif
constexpr int kAlignMergeMaxWg = MOE_ALIGN_MERGE_MAX_WG;   // place workgroups merge the counts themselves up to here

// ------------------------------------------------------------------- count --
// Counts of each expert in each workgroup's chunk: workgroup-major
// (counts[b * E + e], read row-wise by the place workgroups' own merge) or,
// for the scan launch, expert-major (counts[e * G + b]).  The order of the
// slots does not matter here, so a thread reads 4 consecutive ids at a time
// and adds with LDS atomics.
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

// -------------------------------------------------------------------- scan --
// Per expert (one wave each, 16 per workgroup): the exclusive prefix of its
// row of counts over workgroups, in place, and the expert's total.  Lane l
// owns a contiguous run of the row.
__global__ void __launch_bounds__(kAlignThreads)
align_scan_kernel(int32_t* __restrict__ counts, int G, int E, int32_t* __restrict__ totals) {
    const int w = threadIdx.x / kWave, lane = lane_id();
    const int e = blockIdx.x * kAlignWaves + w;
    if (e >= E) return;                            // whole waves
    int32_t* row = counts + (int64_t)e * G;
    const int per = (G + kWave - 1) / kWave;
    const int b0 = lane * per < G ? lane * per : G;
    const int b1 = b0 + per < G ? b0 + per : G;
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += row[b];
    const int incl = wave_incl_scan_i32(sum);
    int run = incl - sum;
    for (int b = b0; b < b1; ++b) {
        const int c = row[b];
        row[b] = run;
        run += c;
    }
    if (lane == kWave - 1) totals[e] = incl;
}

// ------------------------------------------------------------------- place --
// counts: null when G == 1; else the [G,E] counts (totals null: merged here)
// or the per-workgroup bases written by align_scan_kernel (totals given).
template <int R>
__global__ void __launch_bounds__(kAlignThreads)
align_place_kernel(const int32_t* __restrict__ ids, int64_t S, int E, int B, int log2B, int nbits, int64_t C,
                   int G, const int32_t* __restrict__ counts, const int32_t* __restrict__ totals, AlignOut o) {
    extern __shared__ int lds[];
    int* run = lds;                                // [waves][E]
    int* loc = run + kAlignWaves * E;              // [E+1] chunk counts, then local offsets
    int* off = loc + (E + 1);                      // [E+1] aligned offsets
    int* tot = off + (E + 1);                      // [E+1] expert totals
    int* gof = tot + (E + 1);                      // [E+1] output offset of local position 0
    int* scr = gof + (E + 1);                      // [32]
    uint32_t* chunk = reinterpret_cast<uint32_t*>(scr + 32);   // [1024*R]
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id(), b = blockIdx.x;

    const int64_t c0 = (int64_t)b * (kAlignThreads * R);
    const int wfirst = w * (kWave * R) + lane;     // local index of this thread's first slot
    int ev[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t i = c0 + wfirst + j * kWave;
        const int e = i < S ? ids[i] : -1;
        ev[j] = (e >= 0 && e < E) ? e : -1;        // ids outside [0,E) are skipped
    }
    for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) run[i] = 0;

    // this workgroup's base in each expert and the expert totals
    int base_e = 0, all_e = 0;
    if (counts != nullptr && totals != nullptr) {
        if (tid < E) {
            base_e = counts[(int64_t)tid * G + b];
            all_e = totals[tid];
        }
    } else if (counts != nullptr) {
        // every entry of the small [G,E] matrix is loaded in one memory round
        // trip: thread (part, e) sums rows part, part + parts, ... of column e
        // (e fastest across lanes, so each row is read coalesced; e_up and
        // parts are powers of two)
        int e_up = kWave;
        while (e_up < E) e_up <<= 1;
        const int parts = kAlignThreads / e_up, e = tid & (e_up - 1), part = tid / e_up;
        constexpr int kBatch = 16;
        int before = 0, all = 0;
        if (e < E) {
            for (int bb0 = part; bb0 < G; bb0 += kBatch * parts) {
                int c[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int bb = bb0 + u * parts;
                    c[u] = bb < G ? counts[(int64_t)bb * E + e] : 0;
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    all += c[u];
                    before += bb0 + u * parts < b ? c[u] : 0;
                }
            }
        }
        int* pb = reinterpret_cast<int*>(chunk);   // scratch: chunk is not in use yet
        pb[tid] = before;
        pb[kAlignThreads + tid] = all;
        __syncthreads();
        if (tid < E)
            for (int r = 0; r < parts; ++r) {
                base_e += pb[r * e_up + tid];
                all_e += pb[kAlignThreads + r * e_up + tid];
            }
    }
    __syncthreads();

    // count walk: per wave, the occurrences of each expert in its sub-chunk
    // (order does not matter: LDS atomics)
#pragma unroll
    for (int j = 0; j < R; ++j)
        if (ev[j] >= 0) atomicAdd(&run[w * E + ev[j]], 1);
    __syncthreads();

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
        if (G == 1) all_e = mine;
    }
    int nvalid, ptotal, lo, ex;
    block_excl_scan2(tid < E ? mine : 0, tid < E ? (all_e + B - 1) / B * B : 0, scr, &lo, &ex, &nvalid, &ptotal);
    if (tid < E) {
        loc[tid] = lo;
        off[tid] = ex;
        tot[tid] = all_e;
        gof[tid] = ex + base_e - lo;
    }
    if (tid == 0) off[E] = ptotal;
    __syncthreads();

    write_layout(o, off, tot, E, B, log2B, S, C, (int64_t)b * kAlignThreads + tid, (int64_t)G * kAlignThreads);

    // place walk: every slot to its stable position inside the sorted chunk
    // (ranks among the lanes of a step from ballots; steps in slot order)
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const bool valid = ev[j] >= 0;
        const uint64_t m = same_expert_lanes(valid ? ev[j] : 0, valid, nbits);
        if (valid) {
            const int e = ev[j];
            const int r = popc_below(m);
            const int pos = run[w * E + e];
            chunk[loc[e] + pos + r] = ((uint32_t)e << 16) | (uint32_t)(wfirst + j * kWave);
            if (r == 0) run[w * E + e] = pos + __popcll(m);
        }
    }
    __syncthreads();

    // coalesced write-out: position idx of the sorted chunk is slot c0 + local
    for (int idx = tid; idx < nvalid; idx += kAlignThreads) {
        const uint32_t v = chunk[idx];
        o.sorted[gof[v >> 16] + idx] = (int32_t)(c0 + (v & 0xFFFFu));
    }
}

// ------------------------------------------------------------------- host --
int align_nbits(int E) {
    int n = 0;
    while ((1 << n) < E) ++n;
    return n;
}

static int align_max_r(int E) {
    int r = kAlignMaxR;
    while (r > 1 && align_place_lds_ints(E, r) > kAlignLdsInts) r >>= 1;
    return r;
}

AlignPlan align_plan(int64_t S, int E) {
    AlignPlan p;
    const int rmax = align_max_r(E);
    int r = 1;
    if (S <= (int64_t)kAlignThreads * (rmax < 4 ? rmax : 4)) {
        while ((int64_t)kAlignThreads * r < S) r <<= 1;
        p.G = 1;
    } else {
        r = MOE_ALIGN_MIN_R < 2 ? 2 : MOE_ALIGN_MIN_R;   // the in-kernel merge borrows 2048 ints of the chunk
        while (r < rmax && (S + (int64_t)kAlignThreads * r - 1) / ((int64_t)kAlignThreads * r) > MOE_ALIGN_MAX_WG) r <<= 1;
        p.G = (int)((S + (int64_t)kAlignThreads * r - 1) / ((int64_t)kAlignThreads * r));
    }
    p.R = r;
    p.single = p.G == 1;
    p.scan = p.G > kAlignMergeMaxWg;
    p.chunk = (int64_t)kAlignThreads * r;
    p.workspace_bytes = p.single ? 0 : ((int64_t)p.G * E + (p.scan ? E : 0)) * (int64_t)sizeof(int32_t);
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

template <int R>
static hipError_t align_lds_opt_in() {
    static std::once_flag once[kMaxDevices];
    static hipError_t result[kMaxDevices];
    int dev = 0;
    hipError_t err = current_device(&dev);
    if (err != hipSuccess) return err;
    std::call_once(once[dev], [dev] {
        result[dev] = hipFuncSetAttribute((const void*)align_place_kernel<R>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)(kAlignLdsInts * sizeof(int)));
    });
    return result[dev];
}

template <int R>
static hipError_t launch_align_r(const AlignPlan& plan, const int32_t* ids, int64_t S, int E, int B, int64_t C,
                                 const AlignOut& o, void* workspace, hipStream_t stream) {
    const int nbits = align_nbits(E);
    const size_t lds = (size_t)align_place_lds_ints(E, R) * sizeof(int);
    hipError_t err0 = align_lds_opt_in<R>();
    if (err0 != hipSuccess) return err0;
    int32_t* counts = plan.single ? nullptr : static_cast<int32_t*>(workspace);
    int32_t* totals = plan.scan ? counts + (int64_t)plan.G * E : nullptr;
    if (!plan.single) {
        hipLaunchKernelGGL(align_count_kernel<R>, dim3(plan.G), dim3(kAlignThreads), (size_t)E * sizeof(int),
                           stream, ids, S, E, plan.G, plan.scan ? 1 : 0, counts);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        if (plan.scan) {
            hipLaunchKernelGGL(align_scan_kernel, dim3((E + kAlignWaves - 1) / kAlignWaves), dim3(kAlignThreads),
                               0, stream, counts, plan.G, E, totals);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    int log2B = -1;
    if ((B & (B - 1)) == 0) {
        log2B = 0;
        while ((1 << log2B) < B) ++log2B;
    }
    hipLaunchKernelGGL(align_place_kernel<R>, dim3(plan.G), dim3(kAlignThreads), lds, stream, ids, S, E, B,
                       log2B, nbits, C, plan.G, (const int32_t*)counts, (const int32_t*)totals, o);
    return hipGetLastError();
}

// The no-allocation entry point's scratch: a fixed device array in place of
// the caller's workspace.  Every device holds its own copy at its own
// address; host code uses the address returned by hipGetSymbolAddress, never
// the array's name (which is a host-side stand-in).
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
    const AlignOut o{sorted, expert_ids, post_padded, offsets};
    switch (plan.R) {
        case 1: return launch_align_r<1>(plan, ids, S, E, B, C, o, workspace, stream);
        case 2: return launch_align_r<2>(plan, ids, S, E, B, C, o, workspace, stream);
        case 4: return launch_align_r<4>(plan, ids, S, E, B, C, o, workspace, stream);
        case 8: return launch_align_r<8>(plan, ids, S, E, B, C, o, workspace, stream);
        case 16: return launch_align_r<16>(plan, ids, S, E, B, C, o, workspace, stream);
        case 32: return launch_align_r<32>(plan, ids, S, E, B, C, o, workspace, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
