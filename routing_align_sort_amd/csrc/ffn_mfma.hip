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
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "quant.hpp"

namespace moe {

constexpr int kFfnThreads = 256;
constexpr int kAStepBytes = 128;                // activation bytes of a row per K-step
constexpr int kLdsPitch = kAStepBytes + 16;     // padded LDS row, bytes

// Weight formats of the matrix-core path.  A K-step is 128 activation bytes
// of a row: 64 bf16 or 128 E4M3 elements of the contraction.  The weights
// of a K-step are 128 bytes of a row (bf16, E4M3) or 64 (E2M1: two codes per
// byte), loaded by each lane as Q 16-byte quarters of its half of the row.
enum : int { kWBf16 = 0, kWFp8 = 1, kWFp4 = 2 };
template <int kW>
struct Fmt {
    static constexpr int kBits = kW == kWBf16 ? 16 : kW == kWFp8 ? 8 : 4;
    static constexpr int kBStep = kW == kWFp4 ? 64 : 128;   // weight bytes of a row per K-step
    static constexpr int Q = kBStep / 32;                   // 16-byte quarters per lane and K-step
    static constexpr bool kQuantA = kW != kWBf16;           // E4M3 activations, one scale per row
    static constexpr bool kChanScale = kW == kWFp8;         // one fp32 scale per weight row
    // Packed weight layout (written by moe_prepack_weights): for every expert,
    // N tile, K-step, wave and row set, the 64 lanes' quarters q = 0..Q-1 are
    // stored as Q contiguous 1 KB blocks, so each load instruction of a wave
    // reads 1 KB of consecutive bytes and a wave's K-step is one run.
    static constexpr int kPackWave = 2 * Q * 1024;          // two row sets
    static constexpr int kPackStep = 4 * kPackWave;         // four waves
};
// Packed E8M0 block scales of E2M1 weights: for every expert, N tile, K-step
// and wave, one 4-byte word per lane: the lane's two scale bytes of row set 0
// (low half) and of row set 1 (high half).
constexpr int kPackScaleWaveBytes = 64 * 4;
constexpr int kPackScaleStepBytes = 4 * kPackScaleWaveBytes;

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
// 1: a gate/up tile whose last 32-row subtiles are all padding is computed
// as the smaller tile of its live rows (tiles of 64 and 128 rows).
#ifndef MOE_FFN_LIVE_TILES
#define MOE_FFN_LIVE_TILES 1
#endif


#ifndef MOE_FFN_PIN_LOADS
#define MOE_FFN_PIN_LOADS 1
#endif
// 1: the gate/up GEMM's weight ring is refilled part by part (one
// contraction slice of a K-step at a time) right after that part's MFMAs are
// issued.  Measured: the 512-per-expert gate/up GEMMs 4.7% (bf16) and 5-7%
// (fp8) faster, the Zipf fp8 one 2.5%; the same in the down GEMM (16 K-steps)
// 1.5-5% slower.
#ifndef MOE_FFN_SPLIT_RING
#define MOE_FFN_SPLIT_RING 1
#endif
// the same in the down GEMM of the bf16 128-row tile (measured 557 -> 541 us
// at 512 tokens per expert)
#ifndef MOE_FFN_SPLIT_RING_DOWN
#define MOE_FFN_SPLIT_RING_DOWN 1
#endif
// fp32 slot rows stored two columns per lane (8-byte stores) as bf16 ones are
#ifndef MOE_FFN_PAIR_F32
#define MOE_FFN_PAIR_F32 1
#endif
// the same for the top-1 call's output rows
#ifndef MOE_FFN_PAIR_TOP1
#define MOE_FFN_PAIR_TOP1 1
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
    static constexpr int CPR = kAStepBytes / 16;                  // 16-byte A chunks per row
    static constexpr int ACH = ROWS * CPR;                        // A chunks per K-step
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
// An E2M1 operand (32 codes, element j in bits 4j..4j+3) in the low four
// registers of the operand tuple; the instruction reads only those.
__device__ __forceinline__ i32x8_t as_fp4_operand(uint4 v) {
    i32x8_t r;
    r[0] = (int)v.x; r[1] = (int)v.y; r[2] = (int)v.z; r[3] = (int)v.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

// The shared K loop.  A row m starts at abase + arow[m] * arow_bytes
// (arow[m] < 0: a zero row); brow[ns] is this lane's first weight byte for
// row set ns; nk K-steps; acc[MT][NSUB] accumulates.  E2M1 weights also
// stream their block scales: sptr is this lane's first scale word (below).
// Every address derives from the kernel's global-memory arguments, so all
// loads are global loads (vmcnt only) and waiting for one K-step's
// activations never drains the weight loads already in flight for later
// K-steps.
//
// Contraction order inside a K-step (any permutation works if A and B agree):
// lane half h of the 64-wide weight operand covers the K-step's elements
// [h*KS/2, (h+1)*KS/2), split into consecutive MFMA slices (32 elements for
// E4M3 / E2M1, 8 per lane for bf16) -- so each lane's weight bytes of a
// K-step are one contiguous half of its row's K-step, loaded as 16-byte
// quarters, and its E2M1 block scales (one per 32-element slice) are two
// consecutive bytes of the row's scales.  The activation fragments are read
// from LDS in whatever order pairs them with those weight elements.
template <int kW, bool kPacked, bool kNT, int BM, int NSUB, int PF, int LA, bool kSplit = false>
__device__ __forceinline__ void kloop(const uint8_t* __restrict__ abase, const int* arow, int64_t arow_bytes,
                                      const uint8_t* const (&brow)[NSUB], const uint8_t* const (&srow)[NSUB],
                                      int nk, uint8_t* lds, f32x16_t (&acc)[Tile<BM>::MT][NSUB]) {
    using TL = Tile<BM>;
    using F = Fmt<kW>;
    constexpr int MT = TL::MT;
    constexpr int CPR = TL::CPR;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int half = lane >> 5;
    const int r32 = lane & 31;

    // this thread's A chunks: fixed rows for the whole K loop.  Every row of
    // the MFMA tile is loaded and stored, so the loop holds no lane-dependent
    // condition.  A padding row (-1), and a tile row past the block, reads row
    // 0 instead: rows of the product depend only on their own A row, and the
    // outputs of those rows are never used.
    // Chunk r of this thread is tile row tid/CPR + r*RPS, bytes (tid%CPR)*16:
    // one column, so LDS addresses differ by constants and the global
    // addresses are 32-bit offsets from the uniform base (the activation
    // operand is below 4 GiB, checked on the host).
    static_assert(kFfnThreads % CPR == 0, "chunks of a thread share a column");
    constexpr int RPS = kFfnThreads / CPR;            // tile rows between a thread's chunks
    const int lds_a = (tid / CPR) * kLdsPitch + (tid % CPR) * 16;
    uint32_t aoff[TL::APT];
#pragma unroll
    for (int r = 0; r < TL::APT; ++r) {
        const int m = tid / CPR + r * RPS;
        const int row = m < BM ? arow[m] : -1;
        aoff[r] = (uint32_t)((int64_t)(row >= 0 ? row : 0) * arow_bytes) + (uint32_t)((tid % CPR) * 16);
    }

    // A runs LA K-steps ahead in a ring of LA register sets (LA is 1 or PF+1,
    // so ring slots stay compile-time indices in the loop unrolled by PF+1).
    static_assert(LA == 1 || LA == PF + 1, "activation lookahead must divide the unroll");
    uint4 areg[LA][TL::APT];
    // Weights run PF K-steps ahead.  bf16 / E2M1: Q 16-byte quarters per row
    // set (one MFMA slice each); E4M3: two 32-byte operands, each assembled
    // from two 16-byte loads straight into its register tuple.
    using BOp = typename std::conditional<kW == kWFp8, i32x8_t, uint4>::type;
    constexpr int NB = kW == kWFp8 ? 2 : F::Q;
    BOp breg[PF + 1][NSUB][NB];
    // E2M1: one scale word per K-step, byte 2*ns + kk = row set ns, slice kk
    uint32_t sreg[PF + 1];
    static_assert(kW != kWFp4 || NSUB == 2, "scale words pair two row sets");

    // Loads are issued unconditionally (K-step indices clamped at the end):
    // with a fixed number of loads per K-step the compiler's wait counts can
    // wait for just the oldest loads instead of draining everything in flight.
    auto load_a = [&](uint4 (&dst)[TL::APT], int k) {
#pragma unroll
        for (int r = 0; r < TL::APT; ++r)
            dst[r] = __builtin_bit_cast(uint4, *(const u32x4_t*)(abase + (aoff[r] + (uint32_t)(k * kAStepBytes))));
    };
    auto store_a = [&](const uint4 (&src)[TL::APT], int buf) {
#pragma unroll
        for (int r = 0; r < TL::APT; ++r)
            *(uint4*)(lds + buf * TL::ROWS * kLdsPitch + lds_a + r * RPS * kLdsPitch) = src[r];
    };
    constexpr int64_t kB = kPacked ? F::kPackStep : F::kBStep;      // per K-step
    constexpr int qB = kPacked ? 1024 : 16;                           // per quarter
    auto load_b = [&](BOp (&dst)[NSUB][NB], uint32_t& sdst, int k) {
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns) {
            const uint8_t* src = brow[ns] + (int64_t)k * kB;
            if constexpr (kW == kWFp8) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const uint4 lo = load_weight<kNT>(src + (2 * j) * qB);
                    const uint4 hi = load_weight<kNT>(src + (2 * j + 1) * qB);
                    dst[ns][j] = as_i32x8(lo, hi);
                }
            } else {
#pragma unroll
                for (int q = 0; q < NB; ++q) dst[ns][q] = load_weight<kNT>(src + q * qB);
            }
        }
        if constexpr (kW == kWFp4) {
            if constexpr (kPacked) {
                sdst = *(const uint32_t*)(srow[0] + (int64_t)k * kPackScaleStepBytes);
            } else {
                const uint32_t s0 = *(const uint16_t*)(srow[0] + (int64_t)k * 4);
                const uint32_t s1 = *(const uint16_t*)(srow[1] + (int64_t)k * 4);
                sdst = s0 | (s1 << 16);
            }
        }
    };
    // Part p of a K-step's weights (the operand of slice kk = p of the
    // contraction); the E2M1 scale word comes with the last part.
    auto load_b_part = [&](BOp (&dst)[NSUB][NB], uint32_t& sdst, int k, int p) {
#pragma unroll
        for (int ns = 0; ns < NSUB; ++ns) {
            const uint8_t* src = brow[ns] + (int64_t)k * kB;
            if constexpr (kW == kWFp8) {
                const uint4 lo = load_weight<kNT>(src + (2 * p) * qB);
                const uint4 hi = load_weight<kNT>(src + (2 * p + 1) * qB);
                dst[ns][p] = as_i32x8(lo, hi);
            } else {
                dst[ns][p] = load_weight<kNT>(src + p * qB);
            }
        }
        if constexpr (kW == kWFp4) {
            if (p == NB - 1) {
                if constexpr (kPacked) {
                    sdst = *(const uint32_t*)(srow[0] + (int64_t)k * kPackScaleStepBytes);
                } else {
                    const uint32_t s0 = *(const uint16_t*)(srow[0] + (int64_t)k * 4);
                    const uint32_t s1 = *(const uint16_t*)(srow[1] + (int64_t)k * 4);
                    sdst = s0 | (s1 << 16);
                }
            }
        }
    };
    auto compute = [&](const BOp (&b)[NSUB][NB], uint32_t sc, int buf, int part) {
        const uint8_t* base = lds + buf * TL::ROWS * kLdsPitch + r32 * kLdsPitch + half * (kAStepBytes / 2);
        if constexpr (kW == kWBf16) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (part >= 0 && kk != part) continue;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint4 af = *(const uint4*)(base + mt * 32 * kLdsPitch + kk * 16);
#pragma unroll
                    for (int ns = 0; ns < NSUB; ++ns)
                        acc[mt][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af), as_bf16x8(b[ns][kk]),
                                                                              acc[mt][ns], 0, 0, 0);
                }
            }
        } else if constexpr (kW == kWFp8) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (part >= 0 && kk != part) continue;
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
        } else {
            // E4M3 x E2M1.  Each lane half of the E2M1 operand holds 32
            // consecutive elements (slice kk of its half of the K-step, as
            // for E4M3), but the instruction pairs bytes [0,16) of an E4M3
            // lane half h with elements [16h, 16h+16) of the first E2M1 lane
            // half, and bytes [16,32) with the same range of the second: so
            // the activations come from two 16-byte chunks 64 bytes apart.
            // The weights' block scale of (ns, kk) is byte 2*ns + kk of the
            // scale word (an immediate of the instruction); the activations'
            // scale field is 1.0.
            const uint8_t* abase4 = lds + buf * TL::ROWS * kLdsPitch + r32 * kLdsPitch + half * 16;
            auto slice = [&](auto kkc) {
                constexpr int kk = decltype(kkc)::value;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const i32x8_t af = as_i32x8(*(const uint4*)(abase4 + mt * 32 * kLdsPitch + kk * 32),
                                                *(const uint4*)(abase4 + mt * 32 * kLdsPitch + 64 + kk * 32));
                    acc[mt][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af, as_fp4_operand(b[0][kk]), acc[mt][0], 0, 4, 0, 127, kk, (int)sc);
                    acc[mt][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af, as_fp4_operand(b[1][kk]), acc[mt][1], 0, 4, 0, 127, 2 + kk, (int)sc);
                }
            };
            if (part <= 0) slice(std::integral_constant<int, 0>{});
            if (part < 0 || part == 1) slice(std::integral_constant<int, 1>{});
        }
    };

    // prologue: A steps 0..LA-1 loaded and step 0 stored to LDS, weight steps
    // 0..PF-1 in flight
#pragma unroll
    for (int j = 0; j < LA; ++j) load_a(areg[j], min(j, nk - 1));
    // kSplit (split ring): every slot of the ring is full at the start
    // (steps 0..PF), and each part of a step's slot is refilled with step
    // k+PF+1 as soon as that part's MFMAs are issued, so a weight load is in
    // flight up to (NB-1)/NB of a K-step longer than with a whole-step refill
    // at the start of the next step, in the same registers.  It loads one
    // step more at the start and past the end (clamped), which costs more
    // than it hides in short K loops.
#pragma unroll
    for (int s = 0; s < (kSplit ? PF + 1 : PF); ++s) load_b(breg[s], sreg[s], min(s, nk - 1));
    store_a(areg[0], 0);
    __syncthreads();

    // step k: load A(k+LA) into the slot A(k) left (stored during step k-1),
    // load weights for step k+PF, multiply step k, store A(k+1) to the other
    // LDS buffer.
    for (int k0 = 0; k0 < nk; k0 += PF + 1) {
#pragma unroll
        for (int u = 0; u <= PF; ++u) {
            const int k = k0 + u;
            if (k < nk && kSplit) {
                load_a(areg[u % LA], min(k + LA, nk - 1));
                if (MOE_FFN_PIN_LOADS) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int p = 0; p < NB; ++p) {
                    compute(breg[u], sreg[u], k & 1, p);
                    __builtin_amdgcn_sched_barrier(0);
                    load_b_part(breg[u], sreg[u], min(k + PF + 1, nk - 1), p);
                    __builtin_amdgcn_sched_barrier(0);
                }
                store_a(areg[(u + 1) % LA], (k + 1) & 1);
                __syncthreads();
            } else if (k < nk) {
                load_a(areg[u % LA], min(k + LA, nk - 1));
                load_b(breg[(u + PF) % (PF + 1)], sreg[(u + PF) % (PF + 1)], min(k + PF, nk - 1));
                // keep the loads ahead of this step's MFMAs: left to itself
                // the scheduler sinks them to the end of the step
                if (MOE_FFN_PIN_LOADS) __builtin_amdgcn_sched_barrier(0);
                compute(breg[u], sreg[u], k & 1, -1);
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
// Canonical: row `row` of a [rows, row_bytes] slab, this lane's half of the
// row's first K-step.  Packed: the lane's 16 bytes in the first 1 KB block of
// the (nt, w, ns) run.
template <int kW, bool kPacked>
__device__ __forceinline__ const uint8_t* weight_lane_ptr(const uint8_t* slab, int row, int64_t row_bytes,
                                                          int nt, int w, int ns, int lane) {
    using F = Fmt<kW>;
    if (kPacked) {
        const int64_t nk = row_bytes / F::kBStep;
        return slab + (int64_t)nt * nk * F::kPackStep + w * F::kPackWave + ns * (F::Q * 1024) + lane * 16;
    }
    return slab + (int64_t)row * row_bytes + (lane >> 5) * (F::kBStep / 2);
}

// This lane's first E8M0 scale bytes (nk K-steps of 128 elements; a row has
// nk * 4 scale bytes, the lane's two are those of its half of the K-step).
// Canonical: in row `row` of the [rows, nk*4] scale slab.  Packed: the lane's
// word of (nt, w), which also holds the second row set's pair.
template <bool kPacked>
__device__ __forceinline__ const uint8_t* scale_lane_ptr(const uint8_t* slab, int row, int nk, int nt, int w,
                                                         int lane) {
    if (kPacked) return slab + ((int64_t)nt * nk * 4 + w) * kPackScaleWaveBytes + lane * 4;
    return slab + (int64_t)row * nk * 4 + (lane >> 5) * 2;
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
// E2M1 weights: half the weight registers of E4M3 per K-step in flight.
#ifndef MOE_FFN_FP4_PF
#define MOE_FFN_FP4_PF 2
#endif
#ifndef MOE_FFN_FP4_LA_FULL
#define MOE_FFN_FP4_LA_FULL 1
#endif
#ifndef MOE_FFN_FP4_128_OCC
#define MOE_FFN_FP4_128_OCC 2
#endif
#ifndef MOE_FFN_FP4_128_PF
#define MOE_FFN_FP4_128_PF 1
#endif
#ifndef MOE_FFN_FP4_128_LA
#define MOE_FFN_FP4_128_LA 1
#endif
#ifndef MOE_FFN_FP4_256_PF
#define MOE_FFN_FP4_256_PF 2
#endif
#ifndef MOE_FFN_FP4_256_LA
#define MOE_FFN_FP4_256_LA 0
#endif
template <int kW, int BM>
constexpr int ffn_min_blocks() {
    if (BM >= 256) return 1;
    if (BM == 128)
        return kW == kWFp8 ? MOE_FFN_FP8_128_OCC : kW == kWFp4 ? MOE_FFN_FP4_128_OCC : MOE_FFN_OCC128;
    return 2;
}
template <int kW, int BM>
constexpr int ffn_pf() {
    if (BM >= 256) return kW == kWFp8 ? MOE_FFN_FP8_256_PF : kW == kWFp4 ? MOE_FFN_FP4_256_PF : MOE_FFN_PF256;
    if (BM == 128) return kW == kWFp8 ? MOE_FFN_FP8_128_PF : kW == kWFp4 ? MOE_FFN_FP4_128_PF : MOE_FFN_PF128;
    return kW == kWFp4 ? MOE_FFN_FP4_PF : MOE_FFN_PF;
}
template <int kW, int BM, int PF>
constexpr int ffn_la() {
    const bool full = BM < 128    ? (kW == kWFp4 ? MOE_FFN_FP4_LA_FULL : MOE_FFN_LA_FULL)
                      : BM == 128 ? (kW == kWFp8 ? MOE_FFN_FP8_128_LA : kW == kWFp4 ? MOE_FFN_FP4_128_LA
                                                                                  : MOE_FFN_LA128)
                                  : (kW == kWFp8 ? MOE_FFN_FP8_256_LA : kW == kWFp4 ? MOE_FFN_FP4_256_LA
                                                                                  : MOE_FFN_LA256);
    return full ? PF + 1 : 1;
}

// Live-row gate/up tiles (MOE_FFN_LIVE_TILES): the padding of an M block is a suffix
// (an expert's slots come first in its run), so a block of BM rows whose
// last 32-row subtiles are all padding is computed as the smaller tile of
// its live subtiles, with that tile's weight prefetch depth: the registers
// of the accumulators it does not need hold more weight K-steps in flight.
// Such blocks are the lightly loaded experts', whose weights stream from
// HBM once.
template <int BM>
constexpr bool ffn_live_tiles() {
    return MOE_FFN_LIVE_TILES && (BM == 64 || BM == 128);
}
// Rows of the standard tile whose prefetch tuning a live tile of TB rows takes.
template <int TB>
constexpr int live_tune_rows() {
    return TB <= 64 ? 64 : 128;
}
template <int kW, int TB>
constexpr int live_pf() {
    return ffn_pf<kW, live_tune_rows<TB>()>();
}
template <int kW, int BM, int TB, int PF>
constexpr int live_la() {
    return ffn_la<kW, (TB < BM ? live_tune_rows<TB>() : BM), PF>();
}
// Subtiles of the block whose first row is a row of the block (live(m):
// row m holds a slot; read after the barrier that staged the rows).
template <int BM, typename Live>
__device__ __forceinline__ int live_subtiles(Live live) {
    int n = 0;
#pragma unroll
    for (int j = 0; j < Tile<BM>::MT; ++j) n += live(32 * j) ? 1 : 0;
    return n;
}

// LDS of one workgroup: the activation tile and the per-row tables.
template <int BM>
struct FfnSmem {
    __attribute__((aligned(16))) uint8_t lds[Tile<BM>::LDS_BYTES];
    int arow[BM];
    int slots[BM];
    float rowscale[BM];
    float roww[BM];                                       // top-1 combine weight of the row's slot
};

// Row sets of 32 weight rows per wave: NS = 2 (the default tile) or 4 (a
// wave owns twice the columns; the E4M3 128-row tile at one workgroup per
// CU).  Packed weights are laid out for NS = 2; a wave of the NS = 4 tile
// reads the row sets of two adjacent NS = 2 waves, so both share the layout.
// This lane's first weight byte for gate/up row set j of a wave whose 16*NS
// intermediate columns start at n0: sets [0, NS/2) are gate rows, the rest
// up rows, 32 columns each.
template <int kW, bool kPacked, int NS>
__device__ __forceinline__ const uint8_t* gate_up_lane_ptr(const uint8_t* slab, int64_t wrow, int I, int n0, int j,
                                                           int lane) {
    const int half = j / (NS / 2), c0 = n0 + 32 * (j % (NS / 2));
    return weight_lane_ptr<kW, kPacked>(slab, half * I + c0 + (lane & 31), wrow, c0 / 128, (c0 % 128) / 32, half,
                                        lane);
}

// The gate/up tile after its rows are staged: TB rows of the MFMA tile
// (TB < BM: the rows of the block past TB are padding and are not computed;
// the intermediate's rows past TB are left as they are).
template <int kW, bool kPacked, int BM, int TB, int PF, int NS>
__device__ __forceinline__ void stage1_body(const FfnArgs& a, uint16_t* __restrict__ h_out, const Fp8Ws& q,
                                            int mb, int nt, FfnSmem<BM>& sm) {
    using TL = Tile<TB>;
    using F = Fmt<kW>;
    uint8_t* lds = sm.lds;
    const int* arow = sm.arow;
    const float* rowscale = sm.rowscale;
    const int e = a.expert_ids[mb];
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int H = a.H, I = a.I;
    static_assert(NS == 2 || (NS == 4 && kW != kWFp4), "E2M1 scale words pair two row sets");
    const int n0 = nt * 64 * NS + w * 16 * NS;              // this wave's intermediate columns
    const int r32 = lane & 31;
    const int64_t wrow = (int64_t)H * F::kBits / 8;         // weight bytes of a row
    const int nk = (int)(wrow / F::kBStep);
    const uint8_t* wbase = (const uint8_t*)a.w13 + (int64_t)e * 2 * I * wrow;
    const uint8_t* brow[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) brow[j] = gate_up_lane_ptr<kW, kPacked, NS>(wbase, wrow, I, n0, j, lane);
    const uint8_t* srow[NS] = {};
    if constexpr (kW == kWFp4) {
        const uint8_t* sbase = (const uint8_t*)a.w13_scale + (int64_t)e * 2 * I * nk * 4;
        srow[0] = scale_lane_ptr<kPacked>(sbase, n0 + r32, nk, nt, w, lane);
        srow[1] = scale_lane_ptr<kPacked>(sbase, I + n0 + r32, nk, nt, w, lane);
    }
    f32x16_t acc[TL::MT][NS];
    zero_acc(acc);
    const uint8_t* xs = F::kQuantA ? (const uint8_t*)q.xq : (const uint8_t*)a.x;
    const int64_t xrow = F::kQuantA ? (int64_t)H : (int64_t)H * 2;
    constexpr int LA = live_la<kW, BM, TB, PF>();
    if (stream_weights(a, mb, BM, e))
        kloop<kW, kPacked, true, TB, NS, PF, LA, MOE_FFN_SPLIT_RING>(xs, arow, xrow, brow, srow, nk, lds, acc);
    else
        kloop<kW, kPacked, false, TB, NS, PF, LA, MOE_FFN_SPLIT_RING>(xs, arow, xrow, brow, srow, nk, lds, acc);

#pragma unroll
    for (int sub = 0; sub < NS / 2; ++sub) {
        const int col = n0 + 32 * sub + r32;
        float sg = 1.f, su = 1.f;
        if (F::kChanScale) {
            const float* ws13 = (const float*)a.w13_scale;
            sg = ws13[(int64_t)e * 2 * I + col];
            su = ws13[(int64_t)e * 2 * I + I + col];
        }
#pragma unroll
        for (int mt = 0; mt < TL::MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = mt * 32 + acc_row(i, lane);
                float g = acc[mt][sub][i], u = acc[mt][NS / 2 + sub][i];
                if (F::kQuantA) {
                    const float s = (m < BM) ? rowscale[m] : 0.f;
                    g = g * s * sg;
                    u = u * s * su;
                }
                if (a.save_gu && m < BM) {
                    float* gr = a.save_gu + ((int64_t)mb * BM + m) * 2 * I;
                    gr[col] = g;
                    gr[I + col] = u;
                }
                const float hval = silu_f32(g) * u;
                if constexpr (F::kQuantA) {
                    // row max over this wave's 32 columns, then one atomic per row
                    float mx = fabsf(hval);
#pragma unroll
                    for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
                    if (m < BM) {
                        q.a[((int64_t)mb * BM + m) * I + col] = hval;
                        if (r32 == 0 && mx > 0.f) atomicMax(q.amax + (int64_t)mb * BM + m, __float_as_uint(mx));
                    }
                } else {
                    // non-temporal: the down launch reads h once; measured 25 us
                    // faster at decode, up to 4 at prefill (the fp32 rows of the
                    // fp8 path stay cached: mixed there)
                    if (m < BM)
                        __builtin_nontemporal_store(f32_to_bf16_bits(hval), &h_out[((int64_t)mb * BM + m) * I + col]);
                }
            }
    }
}

// One gate/up tile: M block mb, intermediate columns [nt*64*NS, (nt+1)*64*NS).
template <int kW, bool kPacked, int BM, int PF, int NS = 2>
__device__ __forceinline__ void stage1_tile(const FfnArgs& a, uint16_t* __restrict__ h_out, const Fp8Ws& q,
                                            int mb, int nt, FfnSmem<BM>& sm) {
    using F = Fmt<kW>;
    int* arow = sm.arow;
    float* rowscale = sm.rowscale;
    const int tid = threadIdx.x;
    if (tid < BM) {
        const int slot = a.sorted_ids[(int64_t)mb * BM + tid];
        const bool ok = slot < a.S;
        // row of x: the token, or (x already in the sorted order) the row itself
        const int t = ok ? (a.rows_sorted ? mb * BM + tid : slot / a.K) : 0;
        arow[tid] = ok ? t : -1;                          // -1 = padding
        if (F::kQuantA) rowscale[tid] = ok ? q.sx[t] : 0.f;
    }
    __syncthreads();
    // a tile whose block ends in whole 32-row subtiles of padding runs the
    // smaller tile over its rows (the training forward saves every row's
    // gate/up values, so it keeps the whole tile)
    if constexpr (ffn_live_tiles<BM>()) {
        const int live = a.save_gu ? Tile<BM>::MT : live_subtiles<BM>([&](int m) { return arow[m] >= 0; });
        if (live <= 1) return stage1_body<kW, kPacked, BM, 32, live_pf<kW, 32>(), NS>(a, h_out, q, mb, nt, sm);
        if constexpr (BM >= 128) {
            if (live == 2) return stage1_body<kW, kPacked, BM, 64, live_pf<kW, 64>(), NS>(a, h_out, q, mb, nt, sm);
            if (live == 3) return stage1_body<kW, kPacked, BM, 96, live_pf<kW, 96>(), NS>(a, h_out, q, mb, nt, sm);
        }
    }
    stage1_body<kW, kPacked, BM, BM, PF, NS>(a, h_out, q, mb, nt, sm);
}

// Four row sets per wave hold 256 accumulator registers (all AGPRs) at the
// 128-row tile: one workgroup per CU.
template <int kW, int BM, int NS>
constexpr int ffn_stage_blocks() {
    return NS == 4 ? 1 : ffn_min_blocks<kW, BM>();
}

template <int kW, bool kPacked, int BM, int PF, int NS>
__global__ void __launch_bounds__(kFfnThreads, (ffn_stage_blocks<kW, BM, NS>()))
ffn_stage1(FfnArgs a, uint16_t* __restrict__ h_out, Fp8Ws q, int nN) {
    __shared__ FfnSmem<BM> sm;
    int mb, nt;
    if (!ffn_tile(a.post_padded[0] / BM, nN, &mb, &nt)) return;
    stage1_tile<kW, kPacked, BM, PF, NS>(a, h_out, q, mb, nt, sm);
}

// ------------------------------------------------------------------ stage 2 --
// This lane's first weight byte for down row set j of a wave whose 32*NS
// output columns start at n0 (packed: the NS = 2 wave and set that hold
// those 32 columns).
template <int kW, bool kPacked>
__device__ __forceinline__ const uint8_t* down_lane_ptr(const uint8_t* slab, int64_t wrow, int n0, int j, int lane) {
    const int c0 = n0 + 32 * j;
    return weight_lane_ptr<kW, kPacked>(slab, c0 + (lane & 31), wrow, c0 / 256, (c0 % 256) / 64, (c0 % 64) / 32,
                                        lane);
}

// One down tile: M block mb, output columns [nt*128*NS, (nt+1)*128*NS).
template <int kW, bool kPacked, int BM, int PF, int NS = 2>
__device__ __forceinline__ void stage2_tile(const FfnArgs& a, const uint8_t* __restrict__ h_in,
                                            const float* __restrict__ sa, int mb, int nt, FfnSmem<BM>& sm) {
    using TL = Tile<BM>;
    using F = Fmt<kW>;
    uint8_t* lds = sm.lds;
    int* arow = sm.arow;
    int* slots = sm.slots;
    float* rowscale = sm.rowscale;
    const int e = a.expert_ids[mb];
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
    const int H = a.H, I = a.I;
    if (tid < BM) {
        arow[tid] = mb * BM + tid;                        // sorted row of the intermediate
        const int slot = a.sorted_ids[(int64_t)mb * BM + tid];
        slots[tid] = slot;
        if (F::kQuantA) rowscale[tid] = sa[(int64_t)mb * BM + tid];
        if (a.top1_out) sm.roww[tid] = slot < a.S ? a.top1_w[slot] : 0.f;
    }
    __syncthreads();

    static_assert(NS == 2 || (NS == 4 && kW != kWFp4), "E2M1 scale words pair two row sets");
    const int n0 = nt * 128 * NS + w * 32 * NS;             // this wave's output columns
    const int r32 = lane & 31;
    const int64_t wrow = (int64_t)I * F::kBits / 8;
    const int nk = (int)(wrow / F::kBStep);
    const uint8_t* wbase = (const uint8_t*)a.w2 + (int64_t)e * H * wrow;
    const uint8_t* brow[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) brow[j] = down_lane_ptr<kW, kPacked>(wbase, wrow, n0, j, lane);
    const uint8_t* srow[NS] = {};
    if constexpr (kW == kWFp4) {
        const uint8_t* sbase = (const uint8_t*)a.w2_scale + (int64_t)e * H * nk * 4;
        srow[0] = scale_lane_ptr<kPacked>(sbase, n0 + r32, nk, nt, w, lane);
        srow[1] = scale_lane_ptr<kPacked>(sbase, n0 + 32 + r32, nk, nt, w, lane);
    }
    f32x16_t acc[TL::MT][NS];
    zero_acc(acc);
    const int64_t hrow = F::kQuantA ? (int64_t)I : (int64_t)I * 2;
    // the split ring pays in the down GEMM only for the bf16 128-row tile
    // (32 K-steps of 64 elements; the E4M3 / E2M1 tiles have 16)
    constexpr bool kSplit2 = MOE_FFN_SPLIT_RING_DOWN && kW == kWBf16 && BM == 128 && NS == 2;
    if (stream_weights(a, mb, BM, e))
        kloop<kW, kPacked, true, BM, NS, PF, ffn_la<kW, BM, PF>(), kSplit2>(h_in, arow, hrow, brow, srow, nk, lds,
                                                                           acc);
    else
        kloop<kW, kPacked, false, BM, NS, PF, ffn_la<kW, BM, PF>(), kSplit2>(h_in, arow, hrow, brow, srow, nk, lds,
                                                                            acc);

    float sc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) sc[j] = F::kChanScale ? ((const float*)a.w2_scale)[(int64_t)e * H + n0 + 32 * j + r32]
                                                       : 1.f;
    if (a.y_bf16 || (a.top1_out ? MOE_FFN_PAIR_TOP1 : MOE_FFN_PAIR_F32)) {
        // two columns per store: accumulator registers i and i+1 hold rows r
        // and r+1 of column c; neighbouring lanes swap one value each, so an
        // even lane stores (r, c..c+1) and an odd lane (r+1, c-1..c) -- half
        // the store instructions of one value per lane (bf16: 4 bytes, fp32:
        // 8 bytes).  Top-1: the values are first weighted as the combine
        // weights them, 0 + w * y in fp32.
        const bool odd = lane & 1;
#pragma unroll
        for (int mt = 0; mt < TL::MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const int m0 = mt * 32 + acc_row(i, lane);
                const int m = odd ? m0 + 1 : m0;                  // the row this lane stores
                const float rs0 = F::kQuantA && m0 < BM ? rowscale[m0] : 1.f;
                const float rs1 = F::kQuantA && m0 + 1 < BM ? rowscale[m0 + 1] : 1.f;
                const int slot = m < BM ? slots[m] : a.S;
                const float wt0 = a.top1_out && m0 < BM ? sm.roww[m0] : 0.f;
                const float wt1 = a.top1_out && m0 + 1 < BM ? sm.roww[m0 + 1] : 0.f;
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    float v0 = acc[mt][j][i], v1 = acc[mt][j][i + 1];
                    if (F::kQuantA) {
                        v0 = v0 * rs0 * sc[j];
                        v1 = v1 * rs1 * sc[j];
                    }
                    if (a.top1_out) {
                        float o0 = 0.f, o1 = 0.f;
                        o0 += wt0 * v0;
                        o1 += wt1 * v1;
                        v0 = o0;
                        v1 = o1;
                    }
                    const float x = __shfl_xor(odd ? v0 : v1, 1, kWave);
                    const float lo = odd ? x : v0, hi = odd ? v1 : x;
                    if (slot < a.S) {
                        const int64_t off = (int64_t)slot * H + n0 + 32 * j + (r32 & ~1);
                        if (a.top1_out) {
                            // the layer's output is not read again here:
                            // non-temporal bf16 stores
                            if (a.top1_bf16)
                                __builtin_nontemporal_store(
                                    (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16),
                                    (uint32_t*)((uint16_t*)a.top1_out + off));
                            else
                                *(float2*)((float*)a.top1_out + off) = make_float2(lo, hi);
                        } else if (a.y_bf16) {
                            *(uint32_t*)((uint16_t*)a.y_slots + off) =
                                (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
                        } else {
                            const int64_t yrow = a.rows_sorted ? (int64_t)mb * BM + m : (int64_t)slot;
                            *(float2*)(a.y_slots + yrow * H + n0 + 32 * j + (r32 & ~1)) = make_float2(lo, hi);
                        }
                    }
                }
            }
        return;
    }
#pragma unroll
    for (int mt = 0; mt < TL::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = mt * 32 + acc_row(i, lane);
            if (m < BM) {
                const int slot = slots[m];
                if (slot < a.S) {
                    float y[NS];
#pragma unroll
                    for (int j = 0; j < NS; ++j) {
                        y[j] = acc[mt][j][i];
                        if (F::kQuantA) y[j] = y[j] * rowscale[m] * sc[j];
                    }
                    if (a.top1_out) {
                        // the combine of a token's single slot: 0 + w * y in
                        // fp32, as the separate combine sums it
                        const float wt = sm.roww[m];          // staged with the slot ids
                        const int64_t off = (int64_t)slot * H + n0 + r32;
#pragma unroll
                        for (int j = 0; j < NS; ++j) {
                            float o = 0.f;
                            o += wt * y[j];
                            if (a.top1_bf16) {
                                // the layer's output is not read again here:
                                // non-temporal stores keep it out of the
                                // weight stream's way (3-6 us per layer at
                                // prefill)
                                __builtin_nontemporal_store(f32_to_bf16_bits(o),
                                                            (uint16_t*)a.top1_out + off + 32 * j);
                            } else {
                                ((float*)a.top1_out)[off + 32 * j] = o;
                            }
                        }
                    } else {
                        const int64_t yrow = a.rows_sorted ? (int64_t)mb * BM + m : (int64_t)slot;
                        float* dst = a.y_slots + yrow * H + n0 + r32;
#pragma unroll
                        for (int j = 0; j < NS; ++j) dst[32 * j] = y[j];
                    }
                }
            }
        }
}

// Top-1 combine: a token whose id is outside [0,E) has no slot in the layout,
// so no tile writes its output row; the workgroups of the down launch (every
// one, tile or not) zero those rows.  Thread i of workgroup b checks token
// b + i * gridDim (its id is loaded before the tile and tested after it, so
// the check adds no memory round trip to the tile's start); the flagged
// tokens are shared through LDS and each row is zeroed by the whole
// workgroup with coalesced 16-byte stores.
__device__ __forceinline__ void top1_zero_row(const FfnArgs& a, int64_t t) {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    uint4* row;
    int n;
    if (a.top1_bf16) {
        row = (uint4*)((uint16_t*)a.top1_out + t * a.H);
        n = a.H / 8;
    } else {
        row = (uint4*)((float*)a.top1_out + t * a.H);
        n = a.H / 4;
    }
    for (int h = threadIdx.x; h < n; h += kFfnThreads) row[h] = z;
}

__device__ __forceinline__ void top1_zero_skipped(const FfnArgs& a, int64_t t0, int e0, uint64_t* flag_lds) {
    const int64_t stride = (int64_t)gridDim.x * kFfnThreads;
    const int w = threadIdx.x / kWave;
    // uniform over the workgroup: every pass sees the same base
    for (int64_t base = blockIdx.x; base < a.T; base += stride) {
        const int64_t t = base + (int64_t)threadIdx.x * gridDim.x;
        const int e = t == t0 ? e0 : (t < a.T ? a.top1_ids[t] : 0);
        const uint64_t m = ballot(t < a.T && (e < 0 || e >= a.E));
        if (lane_id() == 0) flag_lds[w] = m;
        __syncthreads();
#pragma unroll
        for (int v = 0; v < kFfnThreads / kWave; ++v) {
            uint64_t f = flag_lds[v];
            while (f) {
                const int l = __builtin_ctzll(f);
                f &= f - 1;
                top1_zero_row(a, base + (int64_t)(v * kWave + l) * gridDim.x);
            }
        }
        __syncthreads();
    }
}

template <int kW, bool kPacked, int BM, int PF, int NS>
__global__ void __launch_bounds__(kFfnThreads, (ffn_stage_blocks<kW, BM, NS>()))
ffn_stage2(FfnArgs a, const uint8_t* __restrict__ h_in, const float* __restrict__ sa, int nN) {
    __shared__ FfnSmem<BM> sm;
    __shared__ uint64_t skip_flags[kFfnThreads / kWave];
    const int64_t t0 = blockIdx.x + (int64_t)threadIdx.x * gridDim.x;   // top-1: first token to check
    int e0 = 0;
    if (a.top1_out && t0 < a.T) e0 = a.top1_ids[t0];
    int mb, nt;
    if (ffn_tile(a.post_padded[0] / BM, nN, &mb, &nt))
        stage2_tile<kW, kPacked, BM, PF, NS>(a, h_in, sa, mb, nt, sm);
    if (a.top1_out) top1_zero_skipped(a, t0, e0, skip_flags);
}

// --------------------------------------------------------- fp8 quantisation --
// One workgroup per token: x bf16 row -> E4M3 codes + scale (quant.hpp).
__global__ void __launch_bounds__(kQuantThreads)
quant_tokens_kernel(const uint16_t* __restrict__ x, int H, uint8_t* __restrict__ xq, float* __restrict__ sx,
                    uint32_t* __restrict__ amax_rows, int64_t C) {
    quant_token_row(x, H, xq, sx, amax_rows, C, blockIdx.x, gridDim.x);
}

// Row r of the fp32 intermediate -> E4M3 codes + scale, by a workgroup of
// kQuantThreads threads.
__device__ __forceinline__ void requant_row(const float* __restrict__ a, const uint32_t* __restrict__ amax_rows,
                                            int I, uint8_t* __restrict__ aq, float* __restrict__ sa, int64_t r) {
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
        // the down GEMM reads the codes once: non-temporal, as the x codes
        __builtin_nontemporal_store(u32x2_t{o.x, o.y}, (u32x2_t*)(aq + r * I + j));
    }
}

// One workgroup per sorted row of the intermediate: fp32 a -> E4M3 + scale.
__global__ void __launch_bounds__(kQuantThreads)
requant_rows_kernel(const float* __restrict__ a, const uint32_t* __restrict__ amax_rows,
                    const int32_t* __restrict__ post_padded, int I, uint8_t* __restrict__ aq,
                    float* __restrict__ sa) {
    const int64_t r = blockIdx.x;
    if (r >= post_padded[0]) return;
    requant_row(a, amax_rows, I, aq, sa, r);
}


// ------------------------------------------------------- one-stage schedule --
// Both GEMMs in one persistent launch.  Workgroups claim tiles from eight
// queues, one per XCD (the M blocks are split into eight contiguous ranges,
// and a queue lists its range's gate/up tiles, then its down tiles), starting
// with the queue of their own XCD and then taking from the others.  A down
// tile of M block mb waits until mb's intermediate is complete: the gate/up
// tile that finishes mb last (a per-block counter) requantises the block's
// rows (E4M3 paths) and raises the block's ready flag.
// Progress: a queue hands out indices in order, so a workgroup that claims a
// down tile of a block finds every gate/up tile of that block already
// claimed by a running workgroup, and gate/up tiles never wait.  Every wait
// is still bounded: past kFusedSpinLimit polls it sets the status word and
// proceeds (the result is then wrong, and the status says so).
// Ordering across XCDs (each has its own L2): every wave waits for its stores
// before the barrier, then one thread writes the L2 back (agent-scope
// release), waits for the write-back, and bumps the counter; a waiter
// invalidates its caches (agent-scope acquire) and waits for that before
// releasing its workgroup.
constexpr int kXcds = 8;
constexpr int kFusedSpinLimit = 1 << 20;
constexpr unsigned kWaitVmem = 0xF70;            // s_waitcnt vmcnt(0)

struct FusedCtl {
    int* claim;        // [kXcds] next index of each queue
    int* done;         // [C/16]  gate/up tiles finished per M block
    int* ready;        // [C/16]  the block's intermediate is complete
    int* status;       // [1]     nonzero: a wait gave up
};

// The XCD this wave runs on (hardware register XCC_ID).
__device__ __forceinline__ int xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcds - 1); }

// Tile idx of a queue holding nb M blocks x nN tiles: groups of GROUP_M
// blocks, M block fastest, as in ffn_tile.
__device__ __forceinline__ void queue_tile(int idx, int nb, int nN, int* mb, int* nt) {
    const int per_group = MOE_FFN_GROUP_M * nN;
    const int g = idx / per_group;
    const int first = g * MOE_FFN_GROUP_M;
    const int gsize = min(nb - first, MOE_FFN_GROUP_M);
    const int r = idx - g * per_group;
    *mb = first + r % gsize;
    *nt = r / gsize;
}

// The BM rows of M block mb: fp32 intermediate -> E4M3 codes + per-row
// scales, by one workgroup, with the same arithmetic as requant_row.  The
// row scales go through LDS first, then every thread converts 8 elements at a
// time across all rows, so many loads are in flight at once.
template <int BM>
__device__ __forceinline__ void requant_block(const Fp8Ws& q, int I, int mb, float* inv_lds) {
    const int tid = threadIdx.x;
    if (tid < BM) {
        const int64_t r = (int64_t)mb * BM + tid;
        const float m = __uint_as_float(q.amax[r]);
        inv_lds[tid] = (m > 0.f) ? 448.0f / m : 0.f;
        q.sa[r] = (m > 0.f) ? m / 448.0f : 1.0f;
    }
    __syncthreads();
    const int per_row = I / 8;
    const float* base = q.a + (int64_t)mb * BM * I;
    uint8_t* obase = q.aq + (int64_t)mb * BM * I;
#pragma unroll 4
    for (int c = tid; c < BM * per_row; c += kFfnThreads) {
        const int i = c / per_row;
        const int64_t off = (int64_t)i * I + (int64_t)(c - i * per_row) * 8;
        const float inv = inv_lds[i];
        const f32x4_t v0 = *(const f32x4_t*)(base + off);
        const f32x4_t v1 = *(const f32x4_t*)(base + off + 4);
        uint2 o;
        o.x = e4m3_pack4(v0[0] * inv, v0[1] * inv, v0[2] * inv, v0[3] * inv);
        o.y = e4m3_pack4(v1[0] * inv, v1[1] * inv, v1[2] * inv, v1[3] * inv);
        *(uint2*)(obase + off) = o;
    }
}

__global__ void __launch_bounds__(256) fused_reset_kernel(FusedCtl c, int nblk) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < kXcds) c.claim[i] = 0;
    if (i == 0) c.status[0] = 0;
    if (i < nblk) {
        c.done[i] = 0;
        c.ready[i] = 0;
    }
}

template <int kW, bool kPacked, int BM, int PF>
__global__ void __launch_bounds__(kFfnThreads, (ffn_min_blocks<kW, BM>()))
ffn_fused(FfnArgs a, uint16_t* __restrict__ h, Fp8Ws q, int nN1, int nN2, FusedCtl ctl) {
    constexpr bool kQuant = Fmt<kW>::kQuantA;
    __shared__ FfnSmem<BM> sm;
    __shared__ int s_idx, s_last, s_next;
    const int nmb = a.post_padded[0] / BM;
    const int home = xcc_id();
    const uint8_t* h_in = kQuant ? q.aq : (const uint8_t*)h;
    int x = home;
    for (;;) {
        const int mb0 = (int)((int64_t)x * nmb / kXcds);
        const int nb = (int)((int64_t)(x + 1) * nmb / kXcds) - mb0;
        const int n1 = nb * nN1, n2 = nb * nN2;
        __syncthreads();                                   // s_idx of the last queue is consumed
        if (threadIdx.x == 0) s_idx = atomicAdd(ctl.claim + x, 1);
        __syncthreads();
        int idx = s_idx;
        while (idx < n1 + n2) {
            // claim the queue's next tile now, so the round trip overlaps this
            // tile.  Within one queue this cannot deadlock: a workgroup that
            // holds a gate/up tile ahead is itself on an earlier gate/up tile
            // (which never waits), and nobody waits on a down tile.
            int ahead = 0;
            if (threadIdx.x == 0) ahead = atomicAdd(ctl.claim + x, 1);
            int mb, nt;
            if (idx < n1) {
                queue_tile(idx, nb, nN1, &mb, &nt);
                mb += mb0;
                stage1_tile<kW, kPacked, BM, PF>(a, h, q, mb, nt, sm);
                __builtin_amdgcn_s_waitcnt(kWaitVmem);    // this wave's stores and atomics are done
                __syncthreads();
                if (threadIdx.x == 0) {
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                    __builtin_amdgcn_s_waitcnt(kWaitVmem);
                    const int old = __hip_atomic_fetch_add(ctl.done + mb, 1, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                    s_last = old == nN1 - 1;
                    if (s_last) {
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                        __builtin_amdgcn_s_waitcnt(kWaitVmem);
                    }
                }
                __syncthreads();
                if (s_last) {
                    if constexpr (kQuant) {
                        requant_block<BM>(q, a.I, mb, sm.rowscale);
                        __builtin_amdgcn_s_waitcnt(kWaitVmem);
                        __syncthreads();
                    }
                    if (threadIdx.x == 0) {
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                        __builtin_amdgcn_s_waitcnt(kWaitVmem);
                        __hip_atomic_store(ctl.ready + mb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            } else {
                queue_tile(idx - n1, nb, nN2, &mb, &nt);
                mb += mb0;
                if (threadIdx.x == 0) {
                    int polls = 0;
                    while (__hip_atomic_load(ctl.ready + mb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
                        if (++polls > kFusedSpinLimit) {
                            atomicOr(ctl.status, 1);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(8);
                    }
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    __builtin_amdgcn_s_waitcnt(kWaitVmem);
                }
                __syncthreads();
                stage2_tile<kW, kPacked, BM, PF>(a, h_in, q.sa, mb, nt, sm);
            }
            __syncthreads();                               // the tile's LDS reads are done
            if (threadIdx.x == 0) s_idx = ahead;
            __syncthreads();
            idx = s_idx;
        }
        // queue x is empty: one look at every queue's counter, then the
        // nearest queue (from home) that still has tiles, or done
        if (threadIdx.x < kWave) {
            bool more = false;
            if (threadIdx.x < kXcds) {
                const int y = threadIdx.x;
                const int nby = (int)((int64_t)(y + 1) * nmb / kXcds) - (int)((int64_t)y * nmb / kXcds);
                more = __hip_atomic_load(ctl.claim + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                       nby * (nN1 + nN2);
            }
            const uint64_t m = __ballot(more);
            if (threadIdx.x == 0) {
                int next = -1;
                for (int p = 1; p <= kXcds && next < 0; ++p)
                    if ((m >> ((home + p) & (kXcds - 1))) & 1) next = (home + p) & (kXcds - 1);
                s_next = next;
            }
        }
        __syncthreads();
        x = s_next;
        if (x < 0) break;
    }
}

// -------------------------------------------------------------------- host --
static inline int64_t align256(int64_t v) { return (v + 255) / 256 * 256; }

static int64_t ffn_base_bytes(int w_dtype, int64_t T, int64_t H, int64_t I, int64_t C) {
    if (w_dtype == 0) return align256(C * I * 4);
    if (w_dtype == 1) return align256(C * I * 2);
    return align256(T * H) + align256(T * 4) + align256(C * I * 4) + align256(C * 4) + align256(C * I) +
           align256(C * 4);
}

// The one-stage schedule's control block: queue counters, status, and two
// words per M block (blocks hold at least 16 rows).
static int64_t fused_ctl_ints(int64_t C) { return kXcds + 8 + 2 * (C / 16 + 1); }

int64_t ffn_workspace_bytes(int w_dtype, int64_t T, int64_t H, int64_t I, int64_t C, int fused) {
    return ffn_base_bytes(w_dtype, T, H, I, C) + (fused ? align256(fused_ctl_ints(C) * 4) : 0);
}

static FusedCtl fused_ctl(void* ws, int w_dtype, int64_t T, int64_t H, int64_t I, int64_t C) {
    int* p = (int*)((uint8_t*)ws + ffn_base_bytes(w_dtype, T, H, I, C));
    FusedCtl c;
    c.claim = p;
    c.status = p + kXcds;
    c.done = p + kXcds + 8;
    c.ready = c.done + (C / 16 + 1);
    return c;
}

// Workgroups of one kernel that fit on the device at once (the persistent grid).
template <typename Kern>
static int resident_workgroups(Kern kern) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFfnThreads, 0) != hipSuccess) return 0;
    return cus * per_cu;
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

QuantArgs ffn_quant_args(void* ws, const void* x, int64_t T, int64_t H, int64_t I, int64_t C) {
    const Fp8Ws q = fp8_ws(ws, T, H, I, C);
    return QuantArgs{static_cast<const uint16_t*>(x), (int)H, q.xq, q.sx, q.amax, C};
}

template <int kW, bool kPacked, int BM>
static hipError_t launch_fused_bm(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev,
                                  int w_dtype) {
    constexpr int PF = ffn_pf<kW, BM>();
    constexpr bool kQuant = Fmt<kW>::kQuantA;
    const int nN1 = a.I / 128, nN2 = a.H / 256;
    const int64_t nblk = a.C / BM;
    const int64_t xrows = a.rows_sorted ? a.C : a.T;
    hipError_t err;
    Fp8Ws q{};
    if ((err = record_stage(ev, 0, stream)) != hipSuccess) return err;
    if (kQuant) {
        q = fp8_ws(ws, xrows, a.H, a.I, a.C);
        if (xrows > 0 && !a.x_quantized)
            hipLaunchKernelGGL(quant_tokens_kernel, dim3((unsigned)xrows), dim3(kQuantThreads), 0, stream,
                               (const uint16_t*)a.x, a.H, q.xq, q.sx, q.amax, a.C);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const FusedCtl ctl = fused_ctl(ws, w_dtype, xrows, a.H, a.I, a.C);
    hipLaunchKernelGGL(fused_reset_kernel, dim3((unsigned)((nblk + 255) / 256 + 1)), dim3(256), 0, stream, ctl,
                       (int)nblk);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = record_stage(ev, 1, stream)) != hipSuccess) return err;
    auto kern = ffn_fused<kW, kPacked, BM, PF>;
    static const int resident = resident_workgroups(kern);
    const int64_t tiles = nblk * (nN1 + nN2);
    const int grid = (int)std::min<int64_t>(tiles, resident > 0 ? resident : 256);
    if (grid > 0)
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kFfnThreads), 0, stream, a, (uint16_t*)ws, q, nN1, nN2, ctl);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // one launch: the gate/up interval covers both GEMMs, the others are empty
    for (int i = 2; i < 5; ++i)
        if ((err = record_stage(ev, i, stream)) != hipSuccess) return err;
    return hipSuccess;
}

// E4M3 at the 128-row tile: four row sets per wave (when the widths divide)
// halve the LDS reads and activation re-reads per MFMA, but leave one wave
// per SIMD: measured at 2048 tokens x top-8 of 32 experts, gate/up 756 us
// against 544 with two row sets, down 394 against 398.  Off by default.
#ifndef MOE_FFN_FP8_NS4
#define MOE_FFN_FP8_NS4 0
#endif
#ifndef MOE_FFN_FP8_NS4_PF
#define MOE_FFN_FP8_NS4_PF 1
#endif

template <int kW, bool kPacked, int BM, int NS>
static hipError_t launch_two_stage(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev);

template <int kW, bool kPacked, int BM>
static hipError_t launch_mfma_bm(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    if (a.fused) return launch_fused_bm<kW, kPacked, BM>(a, ws, stream, ev, kW == kWBf16 ? 1 : kW == kWFp8 ? 2 : 3);
    if constexpr (kW == kWFp8 && BM == 128 && MOE_FFN_FP8_NS4)
        if (a.I % 256 == 0 && a.H % 512 == 0) return launch_two_stage<kW, kPacked, BM, 4>(a, ws, stream, ev);
    return launch_two_stage<kW, kPacked, BM, 2>(a, ws, stream, ev);
}

template <int kW, bool kPacked, int BM, int NS>
static hipError_t launch_two_stage(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    constexpr int PF = NS == 4 ? MOE_FFN_FP8_NS4_PF : ffn_pf<kW, BM>();
    constexpr bool kQuant = Fmt<kW>::kQuantA;
    const int nMB = (int)(a.C / BM);
    const int nN1 = a.I / (64 * NS), nN2 = a.H / (128 * NS);
    const int t1 = nMB * nN1, t2 = nMB * nN2;
    hipError_t err;
    Fp8Ws q{};
    const uint8_t* h_in = static_cast<const uint8_t*>(ws);
    if ((err = record_stage(ev, 0, stream)) != hipSuccess) return err;
    if (kQuant) {
        const int64_t xrows = a.rows_sorted ? a.C : a.T;         // rows of x
        q = fp8_ws(ws, xrows, a.H, a.I, a.C);
        if (xrows > 0 && !a.x_quantized)
            hipLaunchKernelGGL(quant_tokens_kernel, dim3((unsigned)xrows), dim3(kQuantThreads), 0, stream,
                               (const uint16_t*)a.x, a.H, q.xq, q.sx, q.amax, a.C);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        h_in = q.aq;
    }
    if ((err = record_stage(ev, 1, stream)) != hipSuccess) return err;
    if (t1 > 0)
        hipLaunchKernelGGL((ffn_stage1<kW, kPacked, BM, PF, NS>), dim3(t1), dim3(kFfnThreads), 0, stream, a,
                           (uint16_t*)ws, q, nN1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = record_stage(ev, 2, stream)) != hipSuccess) return err;
    if (kQuant && a.C > 0) {
        hipLaunchKernelGGL(requant_rows_kernel, dim3((unsigned)a.C), dim3(kQuantThreads), 0, stream,
                           (const float*)q.a, (const uint32_t*)q.amax, a.post_padded, a.I, q.aq, q.sa);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = record_stage(ev, 3, stream)) != hipSuccess) return err;
    if (t2 > 0)
        hipLaunchKernelGGL((ffn_stage2<kW, kPacked, BM, PF, NS>), dim3(t2), dim3(kFfnThreads), 0, stream, a,
                           h_in, (const float*)q.sa, nN2);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return record_stage(ev, 4, stream);
}

template <int kW, bool kPacked>
static hipError_t launch_mfma_layout(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    switch (a.B) {
        case 16: return launch_mfma_bm<kW, kPacked, 16>(a, ws, stream, ev);
        case 32: return launch_mfma_bm<kW, kPacked, 32>(a, ws, stream, ev);
        case 64: return launch_mfma_bm<kW, kPacked, 64>(a, ws, stream, ev);
        case 128: return launch_mfma_bm<kW, kPacked, 128>(a, ws, stream, ev);
        case 256: return launch_mfma_bm<kW, kPacked, 256>(a, ws, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

template <int kW>
static hipError_t launch_mfma(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    return a.packed ? launch_mfma_layout<kW, true>(a, ws, stream, ev)
                    : launch_mfma_layout<kW, false>(a, ws, stream, ev);
}

hipError_t launch_ffn_bf16(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    return launch_mfma<kWBf16>(a, ws, stream, ev);
}
hipError_t launch_ffn_fp8(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    return launch_mfma<kWFp8>(a, ws, stream, ev);
}
hipError_t launch_ffn_fp4(const FfnArgs& a, void* ws, hipStream_t stream, hipEvent_t const* ev) {
    return launch_mfma<kWFp4>(a, ws, stream, ev);
}

// ------------------------------------------------------- backward GEMMs --
// Grouped NT GEMM for the backward: C[m][n] = sum_k A[m][k] * B[n][k], bf16
// operands (canonical rows, K contiguous), fp32 results, on the K loop above.
// by_block: group g is M block g of the sorted layout (g < P/BM): A rows
//   g*BM.., B = the block's expert slab (b + expert_ids[g] * b_group), C rows
//   g*BM..; K fixed.
// per expert: group g is expert g with segment [off[g], off[g+1]) of the
//   sorted layout, a contiguous column range of the transposed activations:
//   A rows m (pitch lda) and B rows n (pitch ldb) both start at column
//   off[g]; K = the segment length (a multiple of 64); C = c + g * c_group.
//   An expert with no rows gets zeros.
template <int BM, int PF>
__global__ void __launch_bounds__(kFfnThreads, (ffn_min_blocks<kWBf16, BM>()))
nt_gemm_kernel(NtGemmArgs g) {
    using TL = Tile<BM>;
    __shared__ FfnSmem<BM> sm;
    const int nN = g.N / 256;
    const int mtiles = g.by_block ? 1 : g.M / BM;
    int t = blockIdx.x;
    const int nt = t % nN;
    t /= nN;
    const int mt = t % mtiles;
    const int grp = t / mtiles;
    int64_t a_off, b_off, c_off;
    int K;
    if (g.by_block) {
        if (grp >= g.post_padded[0] / BM) return;
        a_off = (int64_t)grp * BM * g.lda;
        b_off = (int64_t)g.expert_ids[grp] * g.b_group;
        c_off = (int64_t)grp * BM * g.ldc;
        K = g.K;
    } else {
        const int lo = g.offsets[grp], hi = g.offsets[grp + 1];
        a_off = (int64_t)mt * BM * g.lda + lo;
        b_off = lo;
        c_off = (int64_t)grp * g.c_group + (int64_t)mt * BM * g.ldc;
        K = hi - lo;
    }
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id(), r32 = lane & 31;
    if (tid < BM) sm.arow[tid] = tid;
    __syncthreads();
    const int n0 = nt * 256 + w * 64;                       // this wave's output columns
    const uint8_t* bb = (const uint8_t*)(g.b + b_off);
    const uint8_t* const brow[2] = {bb + (int64_t)(n0 + r32) * g.ldb * 2 + (lane >> 5) * 64,
                                    bb + (int64_t)(n0 + 32 + r32) * g.ldb * 2 + (lane >> 5) * 64};
    const uint8_t* const srow[2] = {nullptr, nullptr};
    f32x16_t acc[TL::MT][2];
    zero_acc(acc);
    const int nk = K / 64;                                  // K-steps of 64 bf16 elements
    if (nk > 0)
        kloop<kWBf16, false, false, BM, 2, PF, ffn_la<kWBf16, BM, PF>()>(
            (const uint8_t*)(g.a + a_off), sm.arow, g.lda * 2, brow, srow, nk, sm.lds, acc);
#pragma unroll
    for (int m2 = 0; m2 < TL::MT; ++m2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m2 * 32 + acc_row(i, lane);
            if (m < BM) {
                float* dst = g.c + c_off + (int64_t)m * g.ldc + n0 + r32;
                dst[0] = acc[m2][0][i];
                dst[32] = acc[m2][1][i];
            }
        }
}

// NN form: C[m][n] = sum_k A[m][k] * B[k][n], B in its own [K][N] layout (N
// contiguous), so weight slabs and activation rows need no transpose.  A
// (K contiguous rows) goes through LDS as in kloop; B goes through LDS in
// its natural layout, 64 K-rows x 128 columns per K-step, and each lane reads
// its MFMA operand with two transposing LDS reads (ds_read_b64_tr_b16): in a
// group of 16 lanes, lanes 4q..4q+3 point at the 16 columns of K-row q and
// lane i receives column i of the four rows.  A lane half h of MFMA slice kk
// covers k = 32h + 8kk .. +7 on both operands (the A read of kloop).
#ifndef MOE_NN_EXPERT_PERSISTENT
#define MOE_NN_EXPERT_PERSISTENT 1
#endif
#ifndef MOE_NN_EXPERT_GRID_MULT
#define MOE_NN_EXPERT_GRID_MULT 1
#endif
constexpr int kNnCols = 128;                         // N columns per workgroup: 4 waves x 32
constexpr int kNnPitch = kNnCols + 8;                // B tile row pitch, elements (272 bytes)
constexpr int kNnPF = 2;                             // K-steps of both operands in flight
typedef short v4i16_t __attribute__((ext_vector_type(4)));

template <int BM>
struct NnSmem {
    __attribute__((aligned(16))) uint8_t a[2 * Tile<BM>::ROWS * kLdsPitch];
    __attribute__((aligned(16))) uint16_t b[2][64 * kNnPitch];
};

template <int BM>
__global__ void __launch_bounds__(kFfnThreads, 2) nn_gemm_kernel(NtGemmArgs g) {
    using TL = Tile<BM>;
    constexpr int MT = TL::MT;
    constexpr int CPR = TL::CPR;
    constexpr int RPS = kFfnThreads / CPR;
    constexpr int BCH = 64 * kNnCols / 8 / kFfnThreads;   // B chunks of 16 bytes per thread per K-step
    __shared__ NnSmem<BM> sm;
    const int nN = g.N / kNnCols;
    const int mtiles = g.by_block ? 1 : g.M / BM;
    int t = blockIdx.x;
    const int nt = t % nN;
    t /= nN;
    const int mt0 = t % mtiles;
    const int grp = t / mtiles;
    int64_t a_off, b_off, c_off;
    int K;
    if (g.by_block) {
        if (grp >= g.post_padded[0] / BM) return;
        a_off = (int64_t)grp * BM * g.lda;
        b_off = (int64_t)g.expert_ids[grp] * g.b_group;
        c_off = (int64_t)grp * BM * g.ldc;
        K = g.K;
    } else {
        const int lo = g.offsets[grp], hi = g.offsets[grp + 1];
        a_off = (int64_t)mt0 * BM * g.lda + lo;              // A: transposed activations, columns lo..
        b_off = (int64_t)lo * g.ldb;                          // B: activation rows lo..
        c_off = (int64_t)grp * g.c_group + (int64_t)mt0 * BM * g.ldc;
        K = hi - lo;
    }
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id(), r32 = lane & 31, half = lane >> 5;
    const int nk = K / 64;
    f32x16_t acc[MT];
#pragma unroll
    for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m2][i] = 0.f;

    if (nk > 0) {
        const uint16_t* A = g.a + a_off;
        const uint16_t* Bt = g.b + b_off + nt * kNnCols;
        // A chunks: rows tid/CPR + r*RPS, bytes (tid%CPR)*16 of each 128-byte K-step
        const int lds_a = (tid / CPR) * kLdsPitch + (tid % CPR) * 16;
        int64_t aoff[TL::APT];
#pragma unroll
        for (int r = 0; r < TL::APT; ++r) {
            const int m = tid / CPR + r * RPS;
            aoff[r] = (int64_t)(m < BM ? m : 0) * g.lda * 2 + (tid % CPR) * 16;
        }
        // B chunks: K-row c/16 of the step, columns (c%16)*8 of the tile
        int64_t boff[BCH];
        int lds_b[BCH];
#pragma unroll
        for (int r = 0; r < BCH; ++r) {
            const int c = tid + r * kFfnThreads;
            boff[r] = (int64_t)(c / 16) * g.ldb + (c % 16) * 8;
            lds_b[r] = (c / 16) * kNnPitch + (c % 16) * 8;
        }
        uint4 areg[kNnPF + 1][TL::APT];
        uint4 breg[kNnPF + 1][BCH];
        auto load = [&](uint4 (&ar)[TL::APT], uint4 (&br)[BCH], int k) {
#pragma unroll
            for (int r = 0; r < TL::APT; ++r)
                ar[r] = __builtin_bit_cast(uint4, *(const u32x4_t*)((const uint8_t*)A + aoff[r] + (int64_t)k * 128));
#pragma unroll
            for (int r = 0; r < BCH; ++r)
                br[r] = __builtin_bit_cast(uint4, *(const u32x4_t*)(Bt + boff[r] + (int64_t)k * 64 * g.ldb));
        };
        auto store = [&](const uint4 (&ar)[TL::APT], const uint4 (&br)[BCH], int buf) {
#pragma unroll
            for (int r = 0; r < TL::APT; ++r)
                *(uint4*)(sm.a + buf * TL::ROWS * kLdsPitch + lds_a + r * RPS * kLdsPitch) = ar[r];
#pragma unroll
            for (int r = 0; r < BCH; ++r) *(uint4*)(&sm.b[buf][lds_b[r]]) = br[r];
        };
        // this lane's transposing-read address in the B tile, before the slice offset
        const int grp16 = lane >> 4, q = (lane >> 2) & 3, sl = lane & 3;
        const int b_row0 = (grp16 >> 1) * 32 + q;
        const int b_col = w * 32 + (grp16 & 1) * 16 + 4 * sl;
        auto compute = [&](int buf) {
            const uint8_t* abase = sm.a + buf * TL::ROWS * kLdsPitch + r32 * kLdsPitch + half * 64;
            const uint16_t* bb = sm.b[buf];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16_t*)(bb + (b_row0 + kk * 8) * kNnPitch + b_col));
                const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16_t*)(bb + (b_row0 + kk * 8 + 4) * kNnPitch + b_col));
                uint4 bv;
                bv.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
                bv.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
                bv.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
                bv.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
#pragma unroll
                for (int m2 = 0; m2 < MT; ++m2) {
                    const uint4 af = *(const uint4*)(abase + m2 * 32 * kLdsPitch + kk * 16);
                    acc[m2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af), as_bf16x8(bv), acc[m2], 0, 0, 0);
                }
            }
        };
        // prologue: steps 0..PF-1 in flight, step 0 in LDS
#pragma unroll
        for (int s2 = 0; s2 < kNnPF; ++s2) load(areg[s2], breg[s2], min(s2, nk - 1));
        store(areg[0], breg[0], 0);
        __syncthreads();
        // ring slots are compile-time: step k0+u loads into slot (u+PF)%(PF+1)
        // and stores slot (u+1)%(PF+1)
        static_assert(kNnPF == 2, "the K loop is unrolled by three");
        auto step = [&](int k, auto uc) {
            constexpr int u = decltype(uc)::value;
            constexpr int sl_ld = (u + kNnPF) % (kNnPF + 1), sl_st = (u + 1) % (kNnPF + 1);
            load(areg[sl_ld], breg[sl_ld], min(k + kNnPF, nk - 1));
            if (MOE_FFN_PIN_LOADS) __builtin_amdgcn_sched_barrier(0);
            compute(k & 1);
            store(areg[sl_st], breg[sl_st], (k + 1) & 1);
            __syncthreads();
        };
        for (int k0 = 0; k0 < nk; k0 += kNnPF + 1) {
            step(k0, std::integral_constant<int, 0>{});
            if (k0 + 1 < nk) step(k0 + 1, std::integral_constant<int, 1>{});
            if (k0 + 2 < nk) step(k0 + 2, std::integral_constant<int, 2>{});
        }
    }
    // The product is written once and not read again by this kernel: stores
    // are non-temporal.  Where the tile buffers can hold it, each wave's BM x
    // 32 block goes through LDS first so that a lane writes 16 bytes and a
    // store instruction covers eight 128-byte row segments (the fp32 weight
    // gradients make these launches bound by their writes).
    if constexpr (sizeof(NnSmem<BM>) >= 4 * BM * 32 * sizeof(float)) {
        __syncthreads();
        if (g.c_bf16) {
            // bf16: the workgroup's whole BM x 128 block goes through LDS, so
            // that a row's 256 bytes leave as 16-byte lanes (whole 128-byte
            // lines; a wave's 64-byte half rows had written slower than fp32)
            float* st = reinterpret_cast<float*>(&sm);
#pragma unroll
            for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
                for (int i = 0; i < 16; ++i) st[(m2 * 32 + acc_row(i, lane)) * kNnCols + w * 32 + r32] = acc[m2][i];
            __syncthreads();
            const int c8 = (tid & 15) * 8, r0 = tid >> 4;
#pragma unroll
            for (int j = 0; j < BM / 16; ++j) {
                const int m = j * 16 + r0;
                const f32x4_t lo = *(const f32x4_t*)(st + m * kNnCols + c8);
                const f32x4_t hi = *(const f32x4_t*)(st + m * kNnCols + c8 + 4);
                const u32x4_t u = {(uint32_t)f32_to_bf16_bits(lo[0]) | ((uint32_t)f32_to_bf16_bits(lo[1]) << 16),
                                   (uint32_t)f32_to_bf16_bits(lo[2]) | ((uint32_t)f32_to_bf16_bits(lo[3]) << 16),
                                   (uint32_t)f32_to_bf16_bits(hi[0]) | ((uint32_t)f32_to_bf16_bits(hi[1]) << 16),
                                   (uint32_t)f32_to_bf16_bits(hi[2]) | ((uint32_t)f32_to_bf16_bits(hi[3]) << 16)};
                __builtin_nontemporal_store(
                    u, (u32x4_t*)((uint16_t*)g.c + c_off + (int64_t)m * g.ldc + nt * kNnCols + c8));
            }
            return;
        }
        float* st = reinterpret_cast<float*>(&sm) + w * BM * 32;
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) st[(m2 * 32 + acc_row(i, lane)) * 32 + r32] = acc[m2][i];
        __builtin_amdgcn_wave_barrier();
        const int cq = (lane & 7) * 4;
#pragma unroll
        for (int j = 0; j < BM / 8; ++j) {
            const int m = j * 8 + (lane >> 3);
            const f32x4_t v = *(const f32x4_t*)(st + m * 32 + cq);
            __builtin_nontemporal_store(v, (f32x4_t*)(g.c + c_off + (int64_t)m * g.ldc + nt * kNnCols + w * 32 + cq));
        }
    } else {
        const int n0 = nt * kNnCols + w * 32 + r32;
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t off = c_off + (int64_t)(m2 * 32 + acc_row(i, lane)) * g.ldc + n0;
                if (g.c_bf16) __builtin_nontemporal_store(f32_to_bf16_bits(acc[m2][i]), (uint16_t*)g.c + off);
                else __builtin_nontemporal_store(acc[m2][i], g.c + off);
            }
    }
}

// The per-expert (weight-gradient) form of the NN GEMM with a bf16 product,
// as a persistent kernel.  An expert's K is only its own rows (a K-step or two at prefill),
// so one tile is a short chain: load, one or two K-steps, epilogue.  Here a
// workgroup walks tiles blockIdx.x, +gridDim.x, ...; when a tile's K loop
// ends, the next tile's first K-step is loaded into registers before this
// tile's epilogue runs, so those loads are in flight while its results go
// out.  Vector-memory waits count loads and stores in issue order, so the
// loads are issued before the stores, and both the K-step's move into LDS
// and the expert offsets (kept in LDS, read with no vector-memory wait) sit
// where a wait for the loads does not also wait for this tile's stores.
// Same tiles, same K order and same results as nn_gemm_kernel per expert.
// With fp32 products the launches are bound by their writes and the
// one-tile-per-workgroup kernel is as fast (slightly faster), so it keeps
// that case.
constexpr int kNnExpertMaxGroups = 1024;

template <int BM>
__global__ void __launch_bounds__(kFfnThreads, 2) nn_gemm_expert_kernel(NtGemmArgs g, int tiles, int groups) {
    using TL = Tile<BM>;
    constexpr int MT = TL::MT;
    constexpr int CPR = TL::CPR;
    constexpr int RPS = kFfnThreads / CPR;
    constexpr int BCH = 64 * kNnCols / 8 / kFfnThreads;
    static_assert(TL::ROWS == BM, "every A row of the tile is a row of C");
    static_assert(sizeof(NnSmem<BM>) >= 4 * BM * 32 * sizeof(float), "the epilogue stages through the tile buffers");
    __shared__ NnSmem<BM> sm;
    __shared__ int s_off[kNnExpertMaxGroups + 1];
    const int nN = g.N / kNnCols;
    const int mtiles = g.M / BM;
    const int tid = threadIdx.x, w = tid / kWave, lane = lane_id(), r32 = lane & 31, half = lane >> 5;
    if (blockIdx.x >= tiles) return;                              // uniform per workgroup
    for (int e = tid; e <= groups; e += kFfnThreads) s_off[e] = g.offsets[e];
    // per-thread chunk offsets in bytes within one K-step, the same for every
    // tile (the host checks that BM rows of A and 64 rows of B span under 2^31
    // bytes)
    const int lds_a = (tid / CPR) * kLdsPitch + (tid % CPR) * 16;
    uint32_t aoff[TL::APT];
#pragma unroll
    for (int r = 0; r < TL::APT; ++r) aoff[r] = (uint32_t)((tid / CPR + r * RPS) * g.lda * 2 + (tid % CPR) * 16);
    uint32_t boff[BCH];
    int lds_b[BCH];
#pragma unroll
    for (int r = 0; r < BCH; ++r) {
        const int c = tid + r * kFfnThreads;
        boff[r] = (uint32_t)(((c / 16) * g.ldb + (c % 16) * 8) * 2);
        lds_b[r] = (c / 16) * kNnPitch + (c % 16) * 8;
    }
    const int64_t bstep = (int64_t)g.ldb * 128;                  // bytes per 64 B rows
    const int grp16 = lane >> 4, q = (lane >> 2) & 3, sl = lane & 3;
    const int b_row0 = (grp16 >> 1) * 32 + q;
    const int b_col = w * 32 + (grp16 & 1) * 16 + 4 * sl;
    __syncthreads();                                              // s_off

    struct TileRef {
        const uint8_t* A;
        const uint8_t* Bt;
        int64_t c_off;
        int nt, nk;
    };
    auto tile_ref = [&](int tile) {
        TileRef r;
        int t = tile;
        r.nt = t % nN;
        t /= nN;
        const int mt0 = t % mtiles, grp = t / mtiles;
        const int lo = __builtin_amdgcn_readfirstlane(s_off[grp]);
        const int hi = __builtin_amdgcn_readfirstlane(s_off[grp + 1]);
        r.A = (const uint8_t*)(g.a + (int64_t)mt0 * BM * g.lda + lo);          // transposed activations
        r.Bt = (const uint8_t*)(g.b + (int64_t)lo * g.ldb + r.nt * kNnCols);   // activation rows lo..
        r.c_off = (int64_t)grp * g.c_group + (int64_t)mt0 * BM * g.ldc;
        r.nk = (hi - lo) / 64;
        return r;
    };
    // two register slots: an expert has a K-step or two, so loads are guarded
    // rather than clamped (a clamped ring would fetch a lone step three times)
    uint4 areg[2][TL::APT];
    uint4 breg[2][BCH];
    auto load = [&](const TileRef& tr, uint4 (&ar)[TL::APT], uint4 (&br)[BCH], int k) {
        const uint8_t* a0 = tr.A + (int64_t)k * 128;             // uniform 64-bit bases, 32-bit lane offsets
        const uint8_t* b0 = tr.Bt + (int64_t)k * bstep;
#pragma unroll
        for (int r = 0; r < TL::APT; ++r) ar[r] = __builtin_bit_cast(uint4, *(const u32x4_t*)(a0 + aoff[r]));
#pragma unroll
        for (int r = 0; r < BCH; ++r) br[r] = __builtin_bit_cast(uint4, *(const u32x4_t*)(b0 + boff[r]));
    };
    auto store = [&](const uint4 (&ar)[TL::APT], const uint4 (&br)[BCH], int buf) {
#pragma unroll
        for (int r = 0; r < TL::APT; ++r)
            *(uint4*)(sm.a + buf * TL::ROWS * kLdsPitch + lds_a + r * RPS * kLdsPitch) = ar[r];
#pragma unroll
        for (int r = 0; r < BCH; ++r) *(uint4*)(&sm.b[buf][lds_b[r]]) = br[r];
    };
    f32x16_t acc[MT];
    auto compute = [&](int buf) {
        const uint8_t* abase = sm.a + buf * TL::ROWS * kLdsPitch + r32 * kLdsPitch + half * 64;
        const uint16_t* bb = sm.b[buf];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16_t*)(bb + (b_row0 + kk * 8) * kNnPitch + b_col));
            const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16_t*)(bb + (b_row0 + kk * 8 + 4) * kNnPitch + b_col));
            uint4 bv;
            bv.x = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
            bv.y = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
            bv.z = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
            bv.w = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
#pragma unroll
            for (int m2 = 0; m2 < MT; ++m2) {
                const uint4 af = *(const uint4*)(abase + m2 * 32 * kLdsPitch + kk * 16);
                acc[m2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(af), as_bf16x8(bv), acc[m2], 0, 0, 0);
            }
        }
    };

    // an expert without rows has nothing to load: its slot is zeroed instead,
    // so that the move into LDS (and the wait for the loads) is unconditional
    auto load_first = [&](const TileRef& tr) {
        if (tr.nk > 0) {
            load(tr, areg[0], breg[0], 0);
        } else {
#pragma unroll
            for (int r = 0; r < TL::APT; ++r) areg[0][r] = uint4{0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < BCH; ++r) breg[0][r] = uint4{0, 0, 0, 0};
        }
    };
    // the epilogue, as nn_gemm_kernel's bf16 one: the whole BM x 128 block
    // staged through LDS, 16-byte non-temporal stores of whole rows
    auto epilogue = [&](const TileRef& tr) {
        __syncthreads();                                          // last K-step's reads done
        float* st = reinterpret_cast<float*>(&sm);
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) st[(m2 * 32 + acc_row(i, lane)) * kNnCols + w * 32 + r32] = acc[m2][i];
        __syncthreads();
        const int c8 = (tid & 15) * 8, r0 = tid >> 4;
        uint16_t* cb = (uint16_t*)g.c + tr.c_off + (int64_t)r0 * g.ldc + tr.nt * kNnCols + c8;
#pragma unroll
        for (int j = 0; j < BM / 16; ++j) {
            const int m = j * 16 + r0;
            const f32x4_t lo = *(const f32x4_t*)(st + m * kNnCols + c8);
            const f32x4_t hi = *(const f32x4_t*)(st + m * kNnCols + c8 + 4);
            const u32x4_t u = {(uint32_t)f32_to_bf16_bits(lo[0]) | ((uint32_t)f32_to_bf16_bits(lo[1]) << 16),
                               (uint32_t)f32_to_bf16_bits(lo[2]) | ((uint32_t)f32_to_bf16_bits(lo[3]) << 16),
                               (uint32_t)f32_to_bf16_bits(hi[0]) | ((uint32_t)f32_to_bf16_bits(hi[1]) << 16),
                               (uint32_t)f32_to_bf16_bits(hi[2]) | ((uint32_t)f32_to_bf16_bits(hi[3]) << 16)};
            __builtin_nontemporal_store(u, (u32x4_t*)cb);
            cb += (int64_t)16 * g.ldc;
        }
    };

    int tile = blockIdx.x;
    TileRef cur = tile_ref(tile);
    load_first(cur);
    store(areg[0], breg[0], 0);
    while (true) {
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m2][i] = 0.f;
        __syncthreads();                                          // K-step 0 in LDS buffer 0
        // step k computes from buffer k & 1 while step k + 1 moves from slot
        // (k + 1) & 1 into the other buffer, last read two steps back
        const int nk = cur.nk;
        for (int k0 = 0; k0 < nk; k0 += 2) {
            const bool one = k0 + 1 < nk, two = k0 + 2 < nk;
            if (one) load(cur, areg[1], breg[1], k0 + 1);
            compute(0);
            if (one) {
                store(areg[1], breg[1], 1);
                __syncthreads();
                if (two) load(cur, areg[0], breg[0], k0 + 2);
                compute(1);
                if (two) {
                    store(areg[0], breg[0], 0);
                    __syncthreads();
                }
            }
        }
        const int next = tile + (int)gridDim.x;
        if (next >= tiles) {                                      // the last tile: nothing to prefetch
            epilogue(cur);
            return;
        }
        // the next tile's first K-step is in flight during this epilogue;
        // every path from these loads reaches the move into LDS below, the
        // one place they are waited for
        const TileRef nxt = tile_ref(next);
        load_first(nxt);
        epilogue(cur);
        __syncthreads();                                          // staging reads done
        store(areg[0], breg[0], 0);
        tile = next;
        cur = nxt;
    }
}

template <int BM>
static hipError_t launch_nn_expert_bm(const NtGemmArgs& g, int64_t tiles, int64_t groups, hipStream_t stream) {
    static const int resident = resident_workgroups(nn_gemm_expert_kernel<BM>);   // once per process
    if (resident <= 0) return hipErrorInvalidValue;
    const int64_t grid = std::min<int64_t>(tiles, (int64_t)resident * MOE_NN_EXPERT_GRID_MULT);
    hipLaunchKernelGGL(nn_gemm_expert_kernel<BM>, dim3((unsigned)grid), dim3(kFfnThreads), 0, stream, g,
                       (int)tiles, (int)groups);
    return hipGetLastError();
}

// Whether nn_gemm_expert_kernel's 32-bit chunk offsets and its offset table
// cover this launch.
static bool nn_expert_fits(const NtGemmArgs& g, int BM, int64_t tiles, int64_t groups) {
    return tiles < INT32_MAX && groups <= kNnExpertMaxGroups && (int64_t)BM * g.lda * 2 < ((int64_t)1 << 31) &&
           (int64_t)64 * g.ldb * 2 < ((int64_t)1 << 31);
}

hipError_t launch_nn_gemm(const NtGemmArgs& g, int BM, int64_t groups, hipStream_t stream) {
    const int64_t tiles = groups * (g.by_block ? 1 : g.M / BM) * (g.N / kNnCols);
    if (tiles == 0) return hipSuccess;
    if (!g.by_block && g.c_bf16 && MOE_NN_EXPERT_PERSISTENT && (BM == 64 || BM == 128) &&
        nn_expert_fits(g, BM, tiles, groups))
        return BM == 64 ? launch_nn_expert_bm<64>(g, tiles, groups, stream)
                        : launch_nn_expert_bm<128>(g, tiles, groups, stream);
    switch (BM) {
        case 64: hipLaunchKernelGGL(nn_gemm_kernel<64>, dim3((unsigned)tiles), dim3(kFfnThreads), 0, stream, g); break;
        case 128: hipLaunchKernelGGL(nn_gemm_kernel<128>, dim3((unsigned)tiles), dim3(kFfnThreads), 0, stream, g); break;
        case 256: hipLaunchKernelGGL(nn_gemm_kernel<256>, dim3((unsigned)tiles), dim3(kFfnThreads), 0, stream, g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int BM>
static hipError_t launch_nt_bm(const NtGemmArgs& g, int64_t groups, hipStream_t stream) {
    constexpr int PF = ffn_pf<kWBf16, BM>();
    const int64_t tiles = groups * (g.by_block ? 1 : g.M / BM) * (g.N / 256);
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((nt_gemm_kernel<BM, PF>), dim3((unsigned)tiles), dim3(kFfnThreads), 0, stream, g);
    return hipGetLastError();
}

// groups: the capacity's M blocks (by_block, BM = block_size_m) or the experts
hipError_t launch_nt_gemm(const NtGemmArgs& g, int BM, int64_t groups, hipStream_t stream) {
    switch (BM) {
        case 64: return launch_nt_bm<64>(g, groups, stream);
        case 128: return launch_nt_bm<128>(g, groups, stream);
        case 256: return launch_nt_bm<256>(g, groups, stream);
        default: return hipErrorInvalidValue;
    }
}

// ----------------------------------------------------------------- prepack --
// One 16-byte chunk per thread, walked in packed order (coalesced writes):
// chunk c -> (expert, N tile, K-step, wave, row set, quarter, lane), and the
// canonical row / byte it comes from.  Row of (tile, wave, row set, lane):
// ns * ns_stride + tile * tile_rows + wave * wave_rows + lane % 32.  A K-step
// is 32*Q bytes of a row; lane half h holds bytes [h*16Q, (h+1)*16Q) of it.
__global__ void __launch_bounds__(256)
prepack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t nchunks, int nN, int nk,
               int log2q, int64_t rows_total, int64_t row_bytes, int ns_stride, int tile_rows, int wave_rows) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= nchunks) return;
    const int Q = 1 << log2q;
    const int lane = (int)(c & 63);
    const int q = (int)((c >> 6) & (Q - 1));
    const int ns = (int)((c >> (6 + log2q)) & 1);
    const int w = (int)((c >> (7 + log2q)) & 3);
    const int64_t rest = c >> (9 + log2q);
    const int k = (int)(rest % nk);
    const int t = (int)((rest / nk) % nN);
    const int64_t e = rest / ((int64_t)nk * nN);
    const int64_t row = (int64_t)ns * ns_stride + (int64_t)t * tile_rows + w * wave_rows + (lane & 31);
    const int64_t byte = (int64_t)k * 32 * Q + (lane >> 5) * 16 * Q + q * 16;
    *(uint4*)(dst + c * 16) = *(const uint4*)(src + (e * rows_total + row) * row_bytes + byte);
}

hipError_t launch_prepack(int E, int H, int I, int bits, const void* w13, const void* w2, void* w13p,
                          void* w2p, hipStream_t stream) {
    const int log2q = bits == 4 ? 1 : 2;        // quarters per lane and K-step: 2 (E2M1) or 4
    const int step = 32 << log2q;               // weight bytes of a row per K-step
    // gate/up: rows [0,2I) of H*bits/8 bytes; tiles of 128 intermediate
    // columns; row set 0 = gate rows, 1 = up rows (I further on).
    {
        const int64_t row_bytes = (int64_t)H * bits / 8;
        const int nk = (int)(row_bytes / step), nN = I / 128;
        const int64_t n = (int64_t)E * nN * nk * 4 * 2 * (64 << log2q);
        hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           (const uint8_t*)w13, (uint8_t*)w13p, n, nN, nk, log2q, (int64_t)2 * I, row_bytes, I,
                           128, 32);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // down: rows [0,H) of I*bits/8 bytes; tiles of 256 output columns; a
    // wave's two row sets are adjacent 32-row blocks.
    {
        const int64_t row_bytes = (int64_t)I * bits / 8;
        const int nk = (int)(row_bytes / step), nN = H / 256;
        const int64_t n = (int64_t)E * nN * nk * 4 * 2 * (64 << log2q);
        hipLaunchKernelGGL(prepack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           (const uint8_t*)w2, (uint8_t*)w2p, n, nN, nk, log2q, (int64_t)H, row_bytes, 32, 256,
                           64);
    }
    return hipGetLastError();
}

// E8M0 block scales [rows, nk*4] (nk K-steps of 128 elements) -> one 4-byte
// word per (expert, N tile, K-step, wave, lane), walked in packed order: the
// lane's two scale bytes of its half of the K-step for row set 0, then for
// row set 1 (rows as in the weight packing).
__global__ void __launch_bounds__(256)
prepack_scales_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t nwords, int nN,
                      int nk, int64_t rows_total, int ns_stride, int tile_rows, int wave_rows) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= nwords) return;
    const int lane = (int)(c & 63);
    const int w = (int)((c >> 6) & 3);
    const int64_t rest = c >> 8;
    const int k = (int)(rest % nk);
    const int t = (int)((rest / nk) % nN);
    const int64_t e = rest / ((int64_t)nk * nN);
    const int64_t row0 = (int64_t)t * tile_rows + w * wave_rows + (lane & 31);
    const int64_t byte = (int64_t)k * 4 + (lane >> 5) * 2;
    const uint8_t* p0 = src + (e * rows_total + row0) * nk * 4 + byte;
    const uint8_t* p1 = p0 + (int64_t)ns_stride * nk * 4;
    *(uint32_t*)(dst + c * 4) = (uint32_t)p0[0] | ((uint32_t)p0[1] << 8) | ((uint32_t)p1[0] << 16) |
                                ((uint32_t)p1[1] << 24);
}

hipError_t launch_prepack_scales(int E, int H, int I, const void* s13, const void* s2, void* s13p, void* s2p,
                                 hipStream_t stream) {
    {
        const int nk = H / 128, nN = I / 128;
        const int64_t n = (int64_t)E * nN * nk * (kPackScaleStepBytes / 4);
        hipLaunchKernelGGL(prepack_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           (const uint8_t*)s13, (uint8_t*)s13p, n, nN, nk, (int64_t)2 * I, I, 128, 32);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    {
        const int nk = I / 128, nN = H / 256;
        const int64_t n = (int64_t)E * nN * nk * (kPackScaleStepBytes / 4);
        hipLaunchKernelGGL(prepack_scales_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           (const uint8_t*)s2, (uint8_t*)s2p, n, nN, nk, (int64_t)H, 32, 256, 64);
    }
    return hipGetLastError();
}

}  // namespace moe
