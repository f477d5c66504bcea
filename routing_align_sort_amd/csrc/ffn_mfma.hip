// Block-aligned grouped expert FFN on gfx950 matrix cores: bf16 and a8w8 fp8.
//
// What it computes: "[Feature]: Add more configuration options for MoE
// assembly kernels" (ROCm/aiter issue 1248), "Suggestion Description" -- per
// block of block_size_m rows of one expert, the gate and up projections,
// SiLU(gate) * up, then the down projection; the a8w8 mode with per-token fp8
// activations, fp8 weights and bf16 output; "Estimated Performance Scaling" --
// the block size trades weight reloads against padding rows.  The GC-MoE
// abstract (zhuanzhiai.com) adds the requantisation of the intermediate before
// the second fp8 GEMM.
//
// Design on MI355X
// ----------------
// * Two GEMM launches.  Stage 1 (gate/up + SiLU*up) writes the intermediate in
//   sorted-row order; stage 2 (down) reads it and scatters fp32 rows to
//   y_slots by slot index.  Grids are sized by capacity (C/B blocks); blocks
//   past num_tokens_post_padded exit at once, so nothing is read back to the
//   host and the sequence is graph-capturable.
// * 256-thread workgroups (4 waves, one per SIMD).  bf16 uses
//   v_mfma_f32_32x32x16_bf16, fp8 v_mfma_scale_f32_32x32x64_f8f6f4 (OCP E4M3
//   operands, unit block scales; per-token and per-channel scales are applied
//   in the epilogue).  Stage 1: a wave owns 32 intermediate columns (its 32 gate
//   rows and 32 up rows of W13), a workgroup 128.  Stage 2: a wave owns 64
//   output columns, a workgroup 256.  The M tile is block_size_m rows (at
//   least one 32-row MFMA tile; rows past the block are zero).
// * A K-step is 128 bytes of every row (64 bf16 or 128 fp8 values).  Expert
//   weights stream straight from HBM into MFMA operand registers: each lane
//   reads 64 contiguous bytes of one weight row per K-step, and the
//   contraction index inside a K-step is permuted identically for the A and B
//   operands so those bytes feed the MFMAs as they are.  Loads run PF K-steps
//   ahead in a register ring, keeping enough bytes in flight per CU to stream
//   HBM.  Each weight element is used by exactly one wave, so it never passes
//   through LDS.
// * Activations (the A operand shared by the 4 waves) go through a
//   double-buffered, row-padded LDS tile (144-byte pitch: conflict-free 16-byte
//   MFMA reads), gathered through sorted_token_ids in stage 1.
// * Tiles are dealt so that each XCD gets a contiguous tile range, walked with
//   the N tile fastest: the workgroups of one XCD share the activation rows of
//   a few M blocks in that XCD's L2, and M blocks of one expert stay close in
//   time so repeated weight tiles hit L2 (the pid remapping idea of the AITER
//   section of the dignews.cc page, "AMD GPU ... 7x faster ...").
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kFfnThreads = 256;
constexpr int kStepBytes = 128;                 // bytes of a row per K-step
constexpr int kLdsPitch = kStepBytes + 16;      // padded LDS row, bytes

// K-steps of weights in flight per wave (register ring depth - 1).
#ifndef MOE_FFN_PF
#define MOE_FFN_PF 2
#endif
#ifndef MOE_FFN_PF128            // the 128-row tile: fewer registers, two workgroups per CU
#define MOE_FFN_PF128 1
#endif
// M blocks per tile group: the tiles of GROUP_M consecutive M blocks are dealt
// with the M block fastest, so the workgroups that run together on one XCD
// cover GROUP_M blocks x a few N tiles and share both operands through L2.
#ifndef MOE_FFN_GROUP_M
#define MOE_FFN_GROUP_M 8
#endif

// Packed weight layout (written by moe_prepack_weights): for every expert,
// N tile, K-step, wave and row set, the 64 lanes' 16-byte quarters q = 0..3
// are stored as four contiguous 1 KB blocks, so each load instruction of a
// wave reads 1 KB of consecutive bytes and a wave's K-step is 8 KB in one run.
constexpr int kPackWaveBytes = 2 * 4 * 1024;              // two row sets x four quarters
constexpr int kPackStepBytes = 4 * kPackWaveBytes;        // four waves

#ifndef MOE_FFN_PIN_LOADS
#define MOE_FFN_PIN_LOADS 1
#endif

// Cache policy of the weight loads.  A tile whose expert has a single M block
// in the launch is the only reader of its weights: streaming (non-temporal)
// loads keep those bytes from displacing reusable lines.  Where several M
// blocks of one expert run close together their tiles re-read the same
// weights, and ordinary loads let the repeats hit L2.
// 0 = always ordinary, 1 = always streaming, 2 = chosen per tile as above.
#ifndef MOE_FFN_NT_MODE
#define MOE_FFN_NT_MODE 2
#endif

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool kNT>
__device__ __forceinline__ uint4 load_weight(const uint8_t* p) {
    if constexpr (kNT) return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)p));
    else return *(const uint4*)p;
}

template <int BM>
struct Tile {
    static constexpr int MT = (BM < 32 ? 32 : BM) / 32;         // 32-row MFMA tiles
    static constexpr int ROWS = MT * 32;
    static constexpr int ACH = ROWS * (kStepBytes / 16);         // 16-byte A chunks per K-step
    static constexpr int APT = ACH / kFfnThreads;                // chunks per thread (exact)
    static_assert(ACH % kFfnThreads == 0, "every thread moves whole chunks");
    static constexpr int LDS_BYTES = 2 * ROWS * kLdsPitch;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ i32x8_t as_i32x8(uint4 lo, uint4 hi) {
    i32x8_t r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// The shared K loop.  A row m starts at abase + arow[m] * arow_bytes
// (arow[m] < 0: a zero row); brow[ns] is this lane's first weight byte for
// row set ns; nk K-steps of 128 bytes; acc[MT][NSUB] accumulates.
// Every address derives from the kernel's global-memory arguments, so all
// loads are global loads (vmcnt only) and waiting for one K-step's
// activations never drains the weight loads already in flight for later
// K-steps.
template <bool kFp8, bool kPacked, bool kNT, int BM, int NSUB, int PF, int LA>
__device__ __forceinline__ void kloop(const uint8_t* __restrict__ abase, const int* arow, int64_t arow_bytes,
                                      const uint8_t* const (&brow)[NSUB], int nk,
                                      uint8_t* lds, f32x16_t (&acc)[Tile<BM>::MT][NSUB]) {
    using TL = Tile<BM>;
    constexpr int MT = TL::MT;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int half = lane >> 5;
    const int r32 = lane & 31;

    // this thread's A chunks: fixed rows for the whole K loop.  Every row of
    // the MFMA tile is loaded and stored, so the loop holds no lane-dependent
    // condition.  A padding row (-1), and a tile row past the block, reads row
    // 0 instead: rows of the product depend only on their own A row, and the
    // outputs of those rows are never used.
    const uint8_t* asrc[TL::APT];
#pragma unroll
    for (int r = 0; r < TL::APT; ++r) {
        const int c = tid + r * kFfnThreads;
        const int row = (c >> 3) < BM ? arow[c >> 3] : -1;
        asrc[r] = abase + (int64_t)(row >= 0 ? row : 0) * arow_bytes + (c & 7) * 16;
    }

    // A runs LA K-steps ahead in a ring of LA register sets (LA is 1 or PF+1,
    // so ring slots stay compile-time indices in the loop unrolled by PF+1).
    static_assert(LA == 1 || LA == PF + 1, "activation lookahead must divide the unroll");
    uint4 areg[LA][TL::APT];
    // Weights run PF K-steps ahead.  bf16: four 16-byte MFMA operands per row
    // set; fp8: two 32-byte operands, each assembled from two 16-byte loads
    // straight into its register tuple.
    using BOp = typename std::conditional<kFp8, i32x8_t, uint4>::type;
    constexpr int NB = kFp8 ? 2 : 4;
    BOp breg[PF + 1][NSUB][NB];

    // Loads are issued unconditionally (K-step indices clamped at the end):
    // with a fixed number of loads per K-step the compiler's wait counts can
    // wait for just the oldest loads instead of draining everything in flight.
    auto load_a = [&](uint4 (&dst)[TL::APT], int k) {
#pragma unroll
        for (int r = 0; r < TL::APT; ++r)
            dst[r] = __builtin_bit_cast(uint4, *(const u32x4_t*)(asrc[r] + (int64_t)k * kStepBytes));
    };
    auto store_a = [&](const uint4 (&src)[TL::APT], int buf) {
#pragma unroll
        for (int r = 0; r < TL::APT; ++r) {
            const int c = tid + r * kFfnThreads;
            *(uint4*)(lds + buf * TL::ROWS * kLdsPitch + (c >> 3) * kLdsPitch + (c & 7) * 16) = src[r];
        }
    };
    constexpr int64_t kB = kPacked ? kPackStepBytes : kStepBytes;   // per K-step
    constexpr int qB = kPacked ? 1024 : 16;                           // per quarter
    auto load_b = [&](BOp (&dst)[NSUB][NB], int k) {
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns) {
            const uint8_t* src = brow[ns] + (int64_t)k * kB;
            if constexpr (kFp8) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint4 lo = load_weight<kNT>(src + (2 * j) * qB);
                    const uint4 hi = load_weight<kNT>(src + (2 * j + 1) * qB);
                    dst[ns][j] = as_i32x8(lo, hi);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[ns][q] = load_weight<kNT>(src + q * qB);
            }
        }
    };
    auto compute = [&](const BOp (&b)[NSUB][NB], int buf) {
        const uint8_t* base = lds + buf * TL::ROWS * kLdsPitch + r32 * kLdsPitch + half * 64;
        if constexpr (!kFp8) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint4 af = *(const uint4*)(base + mt * 32 * kLdsPitch + kk * 16);
#pragma unroll
                    for (int ns = 0; ns < NSUB; ++ns) {
                        if constexpr (!kFp8)
                            acc[mt][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                as_bf16x8(af), as_bf16x8(b[ns][kk]), acc[mt][ns], 0, 0, 0);
                    }
                }
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint4 a0 = *(const uint4*)(base + mt * 32 * kLdsPitch + kk * 32);
                    const uint4 a1 = *(const uint4*)(base + mt * 32 * kLdsPitch + kk * 32 + 16);
#pragma unroll
                    for (int ns = 0; ns < NSUB; ++ns)
                        acc[mt][ns] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            as_i32x8(a0, a1), b[ns][kk], acc[mt][ns], 0, 0, 0, 127, 0, 127);
                }
            }
        }
    };

    // prologue: A steps 0..LA-1 loaded and step 0 stored to LDS, weight steps
    // 0..PF-1 in flight
#pragma unroll
    for (int j = 0; j < LA; ++j) load_a(areg[j], min(j, nk - 1));
#pragma unroll
    for (int s = 0; s < PF; ++s) load_b(breg[s], min(s, nk - 1));
    store_a(areg[0], 0);
    __syncthreads();

    // step k: load A(k+LA) into the slot A(k) left (stored during step k-1),
    // load weights for step k+PF, multiply step k, store A(k+1) to the other
    // LDS buffer.
    for (int k0 = 0; k0 < nk; k0 += PF + 1) {
#pragma unroll
        for (int u = 0; u <= PF; ++u) {
            const int k = k0 + u;
            if (k < nk) {
                load_a(areg[u % LA], min(k + LA, nk - 1));
                load_b(breg[(u + PF) % (PF + 1)], min(k + PF, nk - 1));
                // keep the loads ahead of this step's MFMAs: left to itself
                // the scheduler sinks them to the end of the step
                if (MOE_FFN_PIN_LOADS) __builtin_amdgcn_sched_barrier(0);
                compute(breg[u], k & 1);
                // unconditional: after the last step it rewrites the idle
                // buffer with data nobody reads, but a condition here would
                // let the compiler sink the A loads down to this store
                store_a(areg[(u + 1) % LA], (k + 1) & 1);
                __syncthreads();
            }
        }
    }
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

// Row of the 32x32 MFMA accumulator held by this lane in register i.
__device__ __forceinline__ int acc_row(int i, int lane) { return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }

// Tile of this workgroup.  The grid covers the capacity; only the first
// (P/B)*nN workgroups have a tile.  Those -- not the whole grid -- are dealt
// XCD-contiguously, so the real work spreads over all XCDs; inside an XCD's
// range, groups of GROUP_M M blocks are walked M-block fastest.  Returns
// false for a workgroup without a tile.
__device__ __forceinline__ bool ffn_tile(int nmb, int nN, int* mb, int* nt) {
    const int nvalid = nmb * nN;
    if ((int)blockIdx.x >= nvalid) return false;
    const int t = xcd_contiguous_tile(blockIdx.x, nvalid);
    const int per_group = MOE_FFN_GROUP_M * nN;
    const int g = t / per_group;
    const int first = g * MOE_FFN_GROUP_M;
    const int gsize = min(nmb - first, MOE_FFN_GROUP_M);
    const int r = t - g * per_group;
    *mb = first + r % gsize;
    *nt = r / gsize;
    return true;
}

// This lane's first weight byte for row set ns of wave w in N tile nt.
// Canonical: row `row` of a [rows, row_bytes] slab, this lane's 64-byte half.
// Packed: the lane's 16 bytes in the first 1 KB block of the (nt, w, ns) run.
template <bool kPacked>
__device__ __forceinline__ const uint8_t* weight_lane_ptr(const uint8_t* slab, int row, int64_t row_bytes,
                                                          int nt, int w, int ns, int lane) {
    if (kPacked) {
        const int64_t nk = row_bytes / kStepBytes;
        return slab + (int64_t)nt * nk * kPackStepBytes + w * kPackWaveBytes + ns * 4096 + lane * 16;
    }
    return slab + (int64_t)row * row_bytes + (lane >> 5) * 64;
}

template <int MT, int NSUB>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[MT][NSUB]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][ns][i] = 0.f;
}

struct Fp8Ws {
    uint8_t* xq;        // [T,H] E4M3 codes of x
    float* sx;          // [T]   per-token scales
    float* a;           // [C,I] fp32 intermediate
    uint32_t* amax;     // [C]   per-row max |a| (fp32 bits)
    uint8_t* aq;        // [C,I] E4M3 codes of the intermediate
    float* sa;          // [C]   per-row scales
};

// Whether M block mb (of expert e) reads its weights with the streaming policy.
__device__ __forceinline__ bool stream_weights(const FfnArgs& a, int mb, int BM, int e) {
    if (MOE_FFN_NT_MODE == 0) return false;
    if (MOE_FFN_NT_MODE == 1) return true;
    const int nblk = a.post_padded[0] / BM;
    return (mb == 0 || a.expert_ids[mb - 1] != e) && (mb + 1 >= nblk || a.expert_ids[mb + 1] != e);
}

// ------------------------------------------------------------------ stage 1 --
// bf16: h_out is bf16 [C,I].  fp8: writes fp32 a and the row amax.
// Per-tile tuning: workgroups per CU the register budget is sized for, the
// weight K-steps in flight (PF, a register ring of PF + 1 steps) and whether
// the activations also run PF + 1 steps ahead (else one step).  Tiles up to
// 64 rows: two workgroups per CU.  The 128-row tile: 128 accumulator
// registers; two workgroups per CU leave room for one weight step in flight.
// The 256-row tile: 256 accumulator registers (the AGPR half of the file),
// one workgroup per CU.
#ifndef MOE_FFN_OCC128
#define MOE_FFN_OCC128 2
#endif
#ifndef MOE_FFN_LA128
#define MOE_FFN_LA128 0
#endif
#ifndef MOE_FFN_FP8_128_OCC
#define MOE_FFN_FP8_128_OCC 2
#endif
#ifndef MOE_FFN_FP8_128_PF
#define MOE_FFN_FP8_128_PF 1
#endif
#ifndef MOE_FFN_FP8_128_LA
#define MOE_FFN_FP8_128_LA 1
#endif
#ifndef MOE_FFN_PF256
#define MOE_FFN_PF256 2
#endif
#ifndef MOE_FFN_LA256
#define MOE_FFN_LA256 0
#endif
#ifndef MOE_FFN_FP8_256_PF
#define MOE_FFN_FP8_256_PF 1
#endif
#ifndef MOE_FFN_FP8_256_LA
#define MOE_FFN_FP8_256_LA 0
#endif
#ifndef MOE_FFN_LA_FULL
#define MOE_FFN_LA_FULL 1
#endif
template <bool kFp8, int BM>
constexpr int ffn_min_blocks() {
    if (BM >= 256) return 1;
    if (BM == 128) return kFp8 ? MOE_FFN_FP8_128_OCC : MOE_FFN_OCC128;
    return 2;
}
template <bool kFp8, int BM>
constexpr int ffn_pf() {
    if (BM >= 256) return kFp8 ? MOE_FFN_FP8_256_PF : MOE_FFN_PF256;
    if (BM == 128) return kFp8 ? MOE_FFN_FP8_128_PF : MOE_FFN_PF128;
    return MOE_FFN_PF;
}
template <bool kFp8, int BM, int PF>
constexpr int ffn_la() {
    const bool full = BM < 128    ? MOE_FFN_LA_FULL
                      : BM == 128 ? (kFp8 ? MOE_FFN_FP8_128_LA : MOE_FFN_LA128)
                                  : (kFp8 ? MOE_FFN_FP8_256_LA : MOE_FFN_LA256);
    return full ? PF + 1 : 1;
}

template <bool kFp8, bool kPacked, int BM, int PF>
__global__ void __launch_bounds__(kFfnThreads, (ffn_min_blocks<kFp8, BM>()))
ffn_stage1(FfnArgs a, uint16_t* __restrict__ h_out, Fp8Ws q, int nN) {
    using TL = Tile<BM>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[Tile<BM>::LDS_BYTES];
    __shared__ int arow[BM];
    __shared__ float rowscale[BM];
    int mb, nt;
    if (!ffn_tile(a.post_padded[0] / BM, nN, &mb, &nt)) return;
    const int e = a.expert_ids[mb];
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int H = a.H, I = a.I;
    constexpr int esz = kFp8 ? 1 : 2;
    if (tid < BM) {
        const int slot = a.sorted_ids[(int64_t)mb * BM + tid];
        const bool ok = slot < a.S;
        const int t = ok ? slot / a.K : 0;
        arow[tid] = ok ? t : -1;                          // token row of x, -1 = padding
        if (kFp8) rowscale[tid] = ok ? q.sx[t] : 0.f;
    }
    __syncthreads();

    const int n0 = nt * 128 + w * 32;                       // this wave's intermediate columns
    const int r32 = lane & 31;
    const uint8_t* wbase = (const uint8_t*)a.w13 + (int64_t)e * 2 * I * H * esz;
    const uint8_t* const brow[2] = {
        weight_lane_ptr<kPacked>(wbase, n0 + r32, (int64_t)H * esz, nt, w, 0, lane),
        weight_lane_ptr<kPacked>(wbase, I + n0 + r32, (int64_t)H * esz, nt, w, 1, lane)};
    f32x16_t acc[TL::MT][2];
    zero_acc(acc);
    const uint8_t* xs = kFp8 ? (const uint8_t*)q.xq : (const uint8_t*)a.x;
    if (stream_weights(a, mb, BM, e))
        kloop<kFp8, kPacked, true, BM, 2, PF, ffn_la<kFp8, BM, PF>()>(xs, arow, (int64_t)H * esz, brow,
                                                                    H * esz / kStepBytes, lds, acc);
    else
        kloop<kFp8, kPacked, false, BM, 2, PF, ffn_la<kFp8, BM, PF>()>(xs, arow, (int64_t)H * esz, brow,
                                                                     H * esz / kStepBytes, lds, acc);

    const int col = n0 + r32;
    float sg = 1.f, su = 1.f;
    if (kFp8) {
        sg = a.w13_scale[(int64_t)e * 2 * I + col];
        su = a.w13_scale[(int64_t)e * 2 * I + I + col];
    }
#pragma unroll
    for (int mt = 0; mt < TL::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = mt * 32 + acc_row(i, lane);
            float g = acc[mt][0][i], u = acc[mt][1][i];
            if (kFp8) {
                const float s = (m < BM) ? rowscale[m] : 0.f;
                g = g * s * sg;
                u = u * s * su;
            }
            const float hval = silu_f32(g) * u;
            if constexpr (kFp8) {
                // row max over this wave's 32 columns, then one atomic per row
                float mx = fabsf(hval);
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
                if (m < BM) {
                    q.a[((int64_t)mb * BM + m) * I + col] = hval;
                    if (r32 == 0 && mx > 0.f) atomicMax(q.amax + (int64_t)mb * BM + m, __float_as_uint(mx));
                }
            } else {
                if (m < BM) h_out[((int64_t)mb * BM + m) * I + col] = f32_to_bf16_bits(hval);
            }
        }
}

// ------------------------------------------------------------------ stage 2 --
template <bool kFp8, bool kPacked, int BM, int PF>
__global__ void __launch_bounds__(kFfnThreads, (ffn_min_blocks<kFp8, BM>()))
ffn_stage2(FfnArgs a, const uint8_t* __restrict__ h_in, const float* __restrict__ sa, int nN) {
    using TL = Tile<BM>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[Tile<BM>::LDS_BYTES];
    __shared__ int arow[BM];
    __shared__ int slots[BM];
    __shared__ float rowscale[BM];
    int mb, nt;
    if (!ffn_tile(a.post_padded[0] / BM, nN, &mb, &nt)) return;
    const int e = a.expert_ids[mb];
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int H = a.H, I = a.I;
    constexpr int esz = kFp8 ? 1 : 2;
    if (tid < BM) {
        arow[tid] = mb * BM + tid;                        // sorted row of the intermediate
        slots[tid] = a.sorted_ids[(int64_t)mb * BM + tid];
        if (kFp8) rowscale[tid] = sa[(int64_t)mb * BM + tid];
    }
    __syncthreads();

    const int n0 = nt * 256 + w * 64;                       // this wave's output columns
    const int r32 = lane & 31;
    const uint8_t* wbase = (const uint8_t*)a.w2 + (int64_t)e * H * I * esz;
    const uint8_t* const brow[2] = {
        weight_lane_ptr<kPacked>(wbase, n0 + r32, (int64_t)I * esz, nt, w, 0, lane),
        weight_lane_ptr<kPacked>(wbase, n0 + 32 + r32, (int64_t)I * esz, nt, w, 1, lane)};
    f32x16_t acc[TL::MT][2];
    zero_acc(acc);
    if (stream_weights(a, mb, BM, e))
        kloop<kFp8, kPacked, true, BM, 2, PF, ffn_la<kFp8, BM, PF>()>(h_in, arow, (int64_t)I * esz, brow,
                                                                    I * esz / kStepBytes, lds, acc);
    else
        kloop<kFp8, kPacked, false, BM, 2, PF, ffn_la<kFp8, BM, PF>()>(h_in, arow, (int64_t)I * esz, brow,
                                                                     I * esz / kStepBytes, lds, acc);

    float s0 = 1.f, s1 = 1.f;
    if (kFp8) {
        s0 = a.w2_scale[(int64_t)e * H + n0 + r32];
        s1 = a.w2_scale[(int64_t)e * H + n0 + 32 + r32];
    }
#pragma unroll
    for (int mt = 0; mt < TL::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = mt * 32 + acc_row(i, lane);
            if (m < BM) {
                const int slot = slots[m];
                if (slot < a.S) {
                    float y0 = acc[mt][0][i], y1 = acc[mt][1][i];
                    if (kFp8) {
                        const float rs = rowscale[m];
                        y0 = y0 * rs * s0;
                        y1 = y1 * rs * s1;
                    }
                    float* dst = a.y_slots + (int64_t)slot * H + n0 + r32;
                    dst[0] = y0;
                    dst[32] = y1;
                }
            }
        }
}

// --------------------------------------------------------- fp8 quantisation --
// E4M3 code of v (OCP, nearest even); |v| <= 448 by construction (clamped).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    c = fminf(fmaxf(c, -448.f), 448.f);
    d = fminf(fmaxf(d, -448.f), 448.f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

constexpr int kQuantThreads = 256;

__device__ __forceinline__ float block_max(float v, float* lds4) {
    v = wave_max_f32(v);
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) lds4[w] = v;
    __syncthreads();
    float m = lds4[0];
#pragma unroll
    for (int i = 1; i < kQuantThreads / kWave; ++i) m = fmaxf(m, lds4[i]);
    return m;
}

// One workgroup per token: x bf16 row -> E4M3 codes + scale.  Also clears the
// per-row amax of the intermediate for stage 1.
__global__ void __launch_bounds__(kQuantThreads)
quant_tokens_kernel(const uint16_t* __restrict__ x, int H, uint8_t* __restrict__ xq, float* __restrict__ sx,
                    uint32_t* __restrict__ amax_rows, int64_t C) {
    __shared__ float red[kQuantThreads / kWave];
    const int t = blockIdx.x, tid = threadIdx.x;
    for (int64_t r = (int64_t)t * kQuantThreads + tid; r < C; r += (int64_t)gridDim.x * kQuantThreads)
        amax_rows[r] = 0u;
    const uint16_t* row = x + (int64_t)t * H;
    float m = 0.f;
    for (int h = tid * 8; h < H; h += kQuantThreads * 8) {
        const uint4 v = *(const uint4*)(row + h);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m = fmaxf(m, fabsf(bf16_bits_to_f32((uint16_t)(wv[j] & 0xFFFF))));
            m = fmaxf(m, fabsf(bf16_bits_to_f32((uint16_t)(wv[j] >> 16))));
        }
    }
    m = block_max(m, red);
    const float inv = (m > 0.f) ? 448.0f / m : 0.f;
    if (tid == 0) sx[t] = (m > 0.f) ? m / 448.0f : 1.0f;
    for (int h = tid * 8; h < H; h += kQuantThreads * 8) {
        const uint4 v = *(const uint4*)(row + h);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        float f[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = bf16_bits_to_f32((uint16_t)(wv[j] & 0xFFFF)) * inv;
            f[2 * j + 1] = bf16_bits_to_f32((uint16_t)(wv[j] >> 16)) * inv;
        }
        uint2 o;
        o.x = e4m3_pack4(f[0], f[1], f[2], f[3]);
        o.y = e4m3_pack4(f[4], f[5], f[6], f[7]);
        *(uint2*)(xq + (int64_t)t * H + h) = o;
    }
}

// One workgroup per sorted row of the intermediate: fp32 a -> E4M3 + scale.
__global__ void __launch_bounds__(kQuantThreads)
requant_rows_kernel(const float* __restrict__ a, const uint32_t* __restrict__ amax_rows,
                    const int32_t* __restrict__ post_padded, int I, uint8_t* __restrict__ aq,
                    float* __restrict__ sa) {
    const int64_t r = blockIdx.x;
    if (r >= post_padded[0]) return;
    const float m = __uint_as_float(amax_rows[r]);
    const float inv = (m > 0.f) ? 448.0f / m : 0.f;
    if (threadIdx.x == 0) sa[r] = (m > 0.f) ? m / 448.0f : 1.0f;
    const float* row = a + r * I;
    for (int j = threadIdx.x * 8; j < I; j += kQuantThreads * 8) {
        const f32x4_t v0 = *(const f32x4_t*)(row + j);
        const f32x4_t v1 = *(const f32x4_t*)(row + j + 4);
        uint2 o;
        o.x = e4m3_pack4(v0[0] * inv, v0[1] * inv, v0[2] * inv, v0[3] * inv);
        o.y = e4m3_pack4(v1[0] * inv, v1[1] * inv, v1[2] * inv, v1[3] * inv);
        *(uint2*)(aq + r * I + j) = o;
    }
}

// -------------------------------------------------------------------- host --
static inline int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

int64_t ffn_workspace_bytes(int w_dtype, int64_t T, int64_t H, int64_t I, int64_t C) {
    if (w_dtype == 0) return align256(C * I * 4);
    if (w_dtype == 1) return align256(C * I * 2);
    return align256(T * H) + align256(T * 4) + align256(C * I * 4) + align256(C * 4) + align256(C * I) +
           align256(C * 4);
}

static Fp8Ws fp8_ws(void* ws, int64_t T, int64_t H, int64_t I, int64_t C) {
    uint8_t* p = static_cast<uint8_t*>(ws);
    Fp8Ws q;
    q.xq = p; p += align256(T * H);
    q.sx = (float*)p; p += align256(T * 4);
    q.a = (float*)p; p += align256(C * I * 4);
    q.amax = (uint32_t*)p; p += align256(C * 4);
    q.aq = p; p += align256(C * I);
    q.sa = (float*)p;
    return q;
}

template <bool kFp8, bool kPacked, int BM>
static hipError_t launch_mfma_bm(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    constexpr int PF = ffn_pf<kFp8, BM>();
    const int nMB = (int)(a.C / BM);
    const int nN1 = a.I / 128, nN2 = a.H / 256;
    const int t1 = nMB * nN1, t2 = nMB * nN2;
    hipError_t err;
    Fp8Ws q{};
    const uint8_t* h_in = static_cast<const uint8_t*>(ws);
    if ((err = record_stage(ev, 0, stream)) != hipSuccess) return err;
    if (kFp8) {
        q = fp8_ws(ws, a.T, a.H, a.I, a.C);
        if (a.T > 0)
            hipLaunchKernelGGL(quant_tokens_kernel, dim3(a.T), dim3(kQuantThreads), 0, stream,
                               (const uint16_t*)a.x, a.H, q.xq, q.sx, q.amax, a.C);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        h_in = q.aq;
    }
    if ((err = record_stage(ev, 1, stream)) != hipSuccess) return err;
    if (t1 > 0)
        hipLaunchKernelGGL((ffn_stage1<kFp8, kPacked, BM, PF>), dim3(t1), dim3(kFfnThreads), 0, stream, a,
                           (uint16_t*)ws, q, nN1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = record_stage(ev, 2, stream)) != hipSuccess) return err;
    if (kFp8 && a.C > 0) {
        hipLaunchKernelGGL(requant_rows_kernel, dim3((unsigned)a.C), dim3(kQuantThreads), 0, stream,
                           (const float*)q.a, (const uint32_t*)q.amax, a.post_padded, a.I, q.aq, q.sa);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = record_stage(ev, 3, stream)) != hipSuccess) return err;
    if (t2 > 0)
        hipLaunchKernelGGL((ffn_stage2<kFp8, kPacked, BM, PF>), dim3(t2), dim3(kFfnThreads), 0, stream, a,
                           h_in, (const float*)q.sa, nN2);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return record_stage(ev, 4, stream);
}

template <bool kFp8, bool kPacked>
static hipError_t launch_mfma_layout(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    switch (a.B) {
        case 16: return launch_mfma_bm<kFp8, kPacked, 16>(a, ws, stream, ev);
        case 32: return launch_mfma_bm<kFp8, kPacked, 32>(a, ws, stream, ev);
        case 64: return launch_mfma_bm<kFp8, kPacked, 64>(a, ws, stream, ev);
        case 128: return launch_mfma_bm<kFp8, kPacked, 128>(a, ws, stream, ev);
        case 256: return launch_mfma_bm<kFp8, kPacked, 256>(a, ws, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

template <bool kFp8>
static hipError_t launch_mfma(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    return a.packed ? launch_mfma_layout<kFp8, true>(a, ws, stream, ev)
                    : launch_mfma_layout<kFp8, false>(a, ws, stream, ev);
}

hipError_t launch_ffn_bf16(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    return launch_mfma<false>(a, ws, stream, ev);
}
hipError_t launch_ffn_fp8(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    return launch_mfma<true>(a, ws, stream, ev);
}

// ----------------------------------------------------------------- prepack --
// One 16-byte chunk per thread, walked in packed order (coalesced writes):
// chunk c -> (expert, N tile, K-step, wave, row set, quarter, lane), and the
// canonical row / byte it comes from.  Row of (tile, wave, row set, lane):
// ns * ns_stride + tile * tile_rows + wave * wave_rows + lane % 32.
__global__ void __launch_bounds__(256)
prepack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t nchunks, int nN,
               int nk, int64_t rows_total, int64_t row_bytes, int ns_stride, int tile_rows,
               int wave_rows) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= nchunks) return;
    const int lane = (int)(c & 63);
    const int q = (int)((c >> 6) & 3);
    const int ns = (int)((c >> 8) & 1);
    const int w = (int)((c >> 9) & 3);
    const int64_t rest = c >> 11;
    const int k = (int)(rest % nk);
    const int t = (int)((rest / nk) % nN);
    const int64_t e = rest / ((int64_t)nk * nN);
    const int64_t row = (int64_t)ns * ns_stride + (int64_t)t * tile_rows + w * wave_rows + (lane & 31);
    const int64_t byte = (int64_t)k * kStepBytes + (lane >> 5) * 64 + q * 16;
    *(uint4*)(dst + c * 16) = *(const uint4*)(src + (e * rows_total + row) * row_bytes + byte);
}

hipError_t launch_prepack(int E, int H, int I, int esz, const void* w13, const void* w2, void* w13p,
                          void* w2p, hipStream_t stream) {
    // gate/up: rows [0,2I) of H*esz bytes; tiles of 128 intermediate columns;
    // row set 0 = gate rows, 1 = up rows (I further on).
    {
        const int64_t row_bytes = (int64_t)H * esz;
        const int nk = (int)(row_bytes / kStepBytes), nN = I / 128;
        const int64_t n = (int64_t)E * nN * nk * (kPackStepBytes / 16);
        hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           (const uint8_t*)w13, (uint8_t*)w13p, n, nN, nk, (int64_t)2 * I, row_bytes, I, 128,
                           32);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // down: rows [0,H) of I*esz bytes; tiles of 256 output columns; a wave's
    // two row sets are adjacent 32-row blocks.
    {
        const int64_t row_bytes = (int64_t)I * esz;
        const int nk = (int)(row_bytes / kStepBytes), nN = H / 256;
        const int64_t n = (int64_t)E * nN * nk * (kPackStepBytes / 16);
        hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           (const uint8_t*)w2, (uint8_t*)w2p, n, nN, nk, (int64_t)H, row_bytes, 32, 256, 64);
    }
    return hipGetLastError();
}

}  // namespace moe
