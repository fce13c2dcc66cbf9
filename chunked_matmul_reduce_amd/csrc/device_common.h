// Device helpers shared by the gfx950 kernels (tile_kernel.hip, reduce_kernels.hip,
// unfused.hip): the Philox generator of the dropout mask, bf16 unpacking and the fused
// epilogue (bias add, inverted dropout, residual add; round to nearest even, no fused
// multiply-add).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mmar_internal.h"

namespace mmar {

// ------------------------------------------------------------------ Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
// Round: the 64-bit products M0*c0 and M1*c2 split into high / low words; new counter
// (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is bumped by the Weyl increments
// between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
    constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // one 32 x 32 -> 64-bit multiply per product (v_mad_u64_u32), not a separate
        // high and low multiply
        const uint64_t p0 = static_cast<uint64_t>(kM0) * c0;
        const uint64_t p1 = static_cast<uint64_t>(kM1) * c2;
        const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
        const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
        // three-input XORs, one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += kW0;
        k1 += kW1;
    }
    return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One output from v = T + bias: scaled if kept, then the residual added (dropped: the
// residual itself).
__device__ __forceinline__ float epi1_v(float v, float r, uint32_t word, const DropParams& d) {
    const float y = __fmul_rn(v, d.scale);
    const bool keep = (d.drop_all == 0u) && (word >= d.thr);
    return keep ? __fadd_rn(r, y) : r;
}

__device__ __forceinline__ float epi1(float t, float b, float r, uint32_t word,
                                      const DropParams& d) {
    return epi1_v(__fadd_rn(t, b), r, word, d);
}

// Epilogue of four consecutive outputs starting at linear index e (e % 4 == 0; e = m N + n
// for output (m, n) whatever the buffers' leading dimensions): the Philox block at counter
// (lo32(e / 4), hi32(e / 4), offset words) gives the four elements' words.
__device__ __forceinline__ float4 epilogue4(float4 t, uint2 bias, uint2 res, int64_t e,
                                            const DropParams& d) {
    const uint64_t g = static_cast<uint64_t>(e) >> 2;
    const uint4 w = philox4x32_10(static_cast<uint32_t>(g), static_cast<uint32_t>(g >> 32),
                                  d.ctr2, d.ctr3, d.key0, d.key1);
    float4 o;
    o.x = epi1(t.x, bf16_lo(bias.x), bf16_lo(res.x), w.x, d);
    o.y = epi1(t.y, bf16_hi(bias.x), bf16_hi(res.x), w.y, d);
    o.z = epi1(t.z, bf16_lo(bias.y), bf16_lo(res.y), w.z, d);
    o.w = epi1(t.w, bf16_hi(bias.y), bf16_hi(res.y), w.w, d);
    return o;
}

// The same with the bias already added: v = T + bias.
__device__ __forceinline__ float4 epilogue4_v(float4 v, uint2 res, int64_t e, const DropParams& d) {
    const uint64_t g = static_cast<uint64_t>(e) >> 2;
    const uint4 w = philox4x32_10(static_cast<uint32_t>(g), static_cast<uint32_t>(g >> 32),
                                  d.ctr2, d.ctr3, d.key0, d.key1);
    float4 o;
    o.x = epi1_v(v.x, bf16_lo(res.x), w.x, d);
    o.y = epi1_v(v.y, bf16_hi(res.x), w.y, d);
    o.z = epi1_v(v.z, bf16_lo(res.y), w.z, d);
    o.w = epi1_v(v.w, bf16_hi(res.y), w.w, d);
    return o;
}

// GeLU, tanh form (GPT-2's), in fp32, written as v * sigmoid(2u) = v / (1 + 2^w) with
// u = sqrt(2/pi) (v + 0.044715 v^3) and w = -2 u log2(e) = v (K1 + K2 v^2): the same
// function as v/2 (1 + tanh u), without the cancellation of 1 + tanh u for negative v;
// one v_exp_f32 and one v_rcp_f32 (about 1 fp32 unit each) and an explicit FMA.  2^w
// overflowing to +inf gives -0, the limit.
__device__ __forceinline__ float gelu_tanh_f32(float v) {
    constexpr float K1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
    constexpr float K2 = K1 * 0.044715f;
    const float w = v * __builtin_fmaf(K2, v * v, K1);
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(w));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32), first in the low half.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u | ((u >> 16) & 0x8000u);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace mmar
