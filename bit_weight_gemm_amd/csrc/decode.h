// Exact in-register decode of 2-bit ternary codes to f16 pairs (gfx950).
//
// A device code word holds 16 elements; pair s (elements 2s, 2s+1) has its two
// codes at bits 2s and 16+2s.  For s <= 4 the masked word OR 0x6400 in each half
// is the f16 value 1024 + q*4^s (exponent 2^10, code in the fraction).  One packed
// fused multiply-add by 4^-s minus (2^(10-2s) + 1) then gives q - 1 in each half.
// Every intermediate is a small integer or a power-of-two multiple of one, so
// the result is exact for all four codes: 0,1,2,3 -> -1, 0, +1, +2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq2 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// (q-1) for the pair at position P (0..4) of `w` (codes at bits 2P and 16+2P).
template <int P>
__device__ __forceinline__ h2 pair_m1(uint32_t w) {
    static_assert(P >= 0 && P <= 4, "pair position must lie in the f16 fraction");
    const uint32_t t = (w & (0x00030003u << (2 * P))) | 0x64006400u;
    constexpr float inv = 1.0f / float(1 << (2 * P));
    constexpr float off = -float((1 << (10 - 2 * P)) + 1);
    const h2 vi = {(_Float16)inv, (_Float16)inv};
    const h2 vo = {(_Float16)off, (_Float16)off};
    return __builtin_elementwise_fma(as_h2(t), vi, vo);
}

// All 8 pairs of a word: out[s] = (q_{2s} - 1, q_{2s+1} - 1).
__device__ __forceinline__ void word_m1(uint32_t w, h2 out[8]) {
    out[0] = pair_m1<0>(w);
    out[1] = pair_m1<1>(w);
    out[2] = pair_m1<2>(w);
    out[3] = pair_m1<3>(w);
    out[4] = pair_m1<4>(w);
    const uint32_t w6 = w >> 6;  // pairs 5,6,7 move to positions 2,3,4
    out[5] = pair_m1<2>(w6);
    out[6] = pair_m1<3>(w6);
    out[7] = pair_m1<4>(w6);
}

// The 4 pairs of one half-group (elements 8h..8h+7) as an MFMA operand of 8
// consecutive k: shift the word by 8h so the wanted pairs sit at positions 0..3.
__device__ __forceinline__ h8 half_group_m1(uint32_t w, int h) {
    const uint32_t ws = w >> (8 * h);
    const h2 p0 = pair_m1<0>(ws), p1 = pair_m1<1>(ws), p2 = pair_m1<2>(ws), p3 = pair_m1<3>(ws);
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

}  // namespace tq2
