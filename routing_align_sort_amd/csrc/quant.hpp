// Per-token E4M3 quantisation of the activations (a8w8 and MXFP4 paths):
// s = amax|x[t]| / 448 (1 when the row is zero), codes = E4M3 nearest-even of
// x * (448 / amax), saturated to +-448.  What it computes follows the aiter
// issue's "pertokenFp8" a8w8 mode ("[Feature]: Add more configuration options
// for MoE assembly kernels", "Suggestion Description"); the scale formula is
// the plain reading the pages leave open.  Shared by the FFN's own
// quantisation launch and the launch that routes and quantises at once.
#pragma once
#include "common.hpp"

namespace moe {

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
constexpr int kQuantCache = 4;          // 16-byte chunks of a row a thread keeps in registers

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

// Token t's x bf16 row -> E4M3 codes + scale, by one workgroup of
// kQuantThreads threads.  The nb workgroups that quantise the rows (this one
// is number t among them) also clear the per-row amax of the intermediate
// for the gate/up GEMM.
__device__ __forceinline__ void quant_token_row(const uint16_t* __restrict__ x, int H, uint8_t* __restrict__ xq,
                                                float* __restrict__ sx, uint32_t* __restrict__ amax_rows,
                                                int64_t C, int t, int nb) {
    __shared__ float red[kQuantThreads / kWave];
    const int tid = threadIdx.x;
    for (int64_t r = (int64_t)t * kQuantThreads + tid; r < C; r += (int64_t)nb * kQuantThreads)
        amax_rows[r] = 0u;
    const uint16_t* row = x + (int64_t)t * H;
    // rows up to kQuantCache * 8 * kQuantThreads elements stay in registers
    // between the amax and the encoding (one read of the row); longer rows
    // are read twice
    uint4 cache[kQuantCache];
    const bool cached = H <= kQuantCache * 8 * kQuantThreads;
    float m = 0.f;
    auto absmax8 = [&](const uint4 v) {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            m = fmaxf(m, fabsf(bf16_bits_to_f32((uint16_t)(wv[j] & 0xFFFF))));
            m = fmaxf(m, fabsf(bf16_bits_to_f32((uint16_t)(wv[j] >> 16))));
        }
    };
    if (cached) {
#pragma unroll
        for (int c = 0; c < kQuantCache; ++c) {
            const int h = (tid + c * kQuantThreads) * 8;
            cache[c] = h < H ? *(const uint4*)(row + h) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int c = 0; c < kQuantCache; ++c) absmax8(cache[c]);
    } else {
        for (int h = tid * 8; h < H; h += kQuantThreads * 8) absmax8(*(const uint4*)(row + h));
    }
    m = block_max(m, red);
    const float inv = (m > 0.f) ? 448.0f / m : 0.f;
    if (tid == 0) sx[t] = (m > 0.f) ? m / 448.0f : 1.0f;
    auto encode8 = [&](const uint4 v, int h) {
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
        // non-temporal: the gate/up GEMM that reads the codes next streams
        // faster when this kernel leaves no dirty lines behind (8% at 64
        // tokens per expert)
        __builtin_nontemporal_store(u32x2_t{o.x, o.y}, (u32x2_t*)(xq + (int64_t)t * H + h));
    };
    if (cached) {
#pragma unroll
        for (int c = 0; c < kQuantCache; ++c) {
            const int h = (tid + c * kQuantThreads) * 8;
            if (h < H) encode8(cache[c], h);
        }
    } else {
        for (int h = tid * 8; h < H; h += kQuantThreads * 8) encode8(*(const uint4*)(row + h), h);
    }
}


}  // namespace moe
