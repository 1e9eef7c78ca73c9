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

// The f16 exponent pattern 0x6400 in both halves, materialised in a VGPR behind
// an asm statement so the compiler cannot fold it: the masked insert below then
// becomes one v_bfi_b32 (mask in an SGPR, word and pattern in VGPRs) instead of a
// separate AND and OR.  Call once per kernel and pass the value down.
__device__ __forceinline__ uint32_t f16_magic() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m));
    return m;
}

// (q-1) for the pair at position P (0..4) of `w` (codes at bits 2P and 16+2P):
// insert the two codes into 0x6400 (f16 1024 + q*4^P), then one packed FMA.
template <int P>
__device__ __forceinline__ h2 pair_m1(uint32_t w, uint32_t magic) {
    static_assert(P >= 0 && P <= 4, "pair position must lie in the f16 fraction");
    constexpr uint32_t mask = 0x00030003u << (2 * P);
    const uint32_t t = (w & mask) | (magic & ~mask);
    constexpr float inv = 1.0f / float(1 << (2 * P));
    constexpr float off = -float((1 << (10 - 2 * P)) + 1);
    const h2 vi = {(_Float16)inv, (_Float16)inv};
    const h2 vo = {(_Float16)off, (_Float16)off};
    return __builtin_elementwise_fma(as_h2(t), vi, vo);
}

// All 8 pairs of a word: out[s] = (q_{2s} - 1, q_{2s+1} - 1).
__device__ __forceinline__ void word_m1(uint32_t w, uint32_t magic, h2 out[8]) {
    out[0] = pair_m1<0>(w, magic);
    out[1] = pair_m1<1>(w, magic);
    out[2] = pair_m1<2>(w, magic);
    out[3] = pair_m1<3>(w, magic);
    out[4] = pair_m1<4>(w, magic);
    const uint32_t w6 = w >> 6;  // pairs 5,6,7 move to positions 2,3,4
    out[5] = pair_m1<2>(w6, magic);
    out[6] = pair_m1<3>(w6, magic);
    out[7] = pair_m1<4>(w6, magic);
}

// The same decode with its constants in scalar registers, for kernels that
// decode each word once (so nothing is gained by keeping per-position constants
// in vector registers): v_bfi_b32 takes the mask from an SGPR and the word and
// the 0x6400 pattern from VGPRs, and v_pk_fma_f16 takes the factor 4^-P and the
// offset -(2^(10-2P) + 1) from the low and high halves of one SGPR (op_sel).
// Written as inline asm, so only for vector-ALU consumers: the compiler does not
// see these register writes when it spaces MFMA operand reads and writes, so
// MFMA operands come from word_m1 / half_group_m1.
constexpr uint32_t f16_bits(float v) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v); }
template <int P>
__device__ __forceinline__ h2 pair_m1_s(uint32_t w, uint32_t magic) {
    static_assert(P >= 0 && P <= 4, "pair position must lie in the f16 fraction");
    constexpr uint32_t mask = 0x00030003u << (2 * P);
    constexpr uint32_t k = f16_bits(1.0f / float(1 << (2 * P))) | (f16_bits(-float((1 << (10 - 2 * P)) + 1)) << 16);
    uint32_t t, r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(t) : "s"(mask), "v"(w), "v"(magic));
    asm("v_pk_fma_f16 %0, %1, %2, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(t), "s"(k));
    return as_h2(r);
}
static_assert(f16_bits(1.0f / 256.0f) == 0x1C00u && f16_bits(-1025.0f) == 0xE401u, "f16 constants");
__device__ __forceinline__ void word_m1_s(uint32_t w, uint32_t magic, h2 out[8]) {
    out[0] = pair_m1_s<0>(w, magic);
    out[1] = pair_m1_s<1>(w, magic);
    out[2] = pair_m1_s<2>(w, magic);
    out[3] = pair_m1_s<3>(w, magic);
    out[4] = pair_m1_s<4>(w, magic);
    const uint32_t w6 = w >> 6;
    out[5] = pair_m1_s<2>(w6, magic);
    out[6] = pair_m1_s<3>(w6, magic);
    out[7] = pair_m1_s<4>(w6, magic);
}

// The 4 pairs of one half-group (elements 8h..8h+7) as an MFMA operand of 8
// consecutive k: shift the word by 8h so the wanted pairs sit at positions 0..3.
__device__ __forceinline__ h8 half_group_m1(uint32_t w, int h, uint32_t magic) {
    const uint32_t ws = w >> (8 * h);
    const h2 p0 = pair_m1<0>(ws, magic), p1 = pair_m1<1>(ws, magic), p2 = pair_m1<2>(ws, magic),
             p3 = pair_m1<3>(ws, magic);
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}


}  // namespace tq2

namespace tq2 {

// ---- cross-lane helpers (wave64)

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each 16-lane row; every lane of the row ends with the row's total.
// Order: xor 1, xor 2 (quad permutes), then rotate by 4 and by 8 within the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x124>(v);  // row_ror:4
    v += dpp<0x128>(v);  // row_ror:8
    return v;
}

// Exchange of lane halves (v_permlane32_swap_b32): returns the pair after the swap.
__device__ __forceinline__ void swap32(float &a, float &b) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                              false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Exchange of odd/even 16-lane rows (v_permlane16_swap_b32).
__device__ __forceinline__ void swap16(float &a, float &b) {
    auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                              false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Which operand's row a lane keeps after swap32/swap16 (0: first, 1: second),
// found by pushing the row tags 0 and 1 through the same exchange.
__device__ __forceinline__ int kept32() {
    auto r = __builtin_amdgcn_permlane32_swap(0u, 1u, false, false);
    return (int)(uint32_t)r[0];
}
__device__ __forceinline__ int kept16() {
    auto r = __builtin_amdgcn_permlane16_swap(0u, 1u, false, false);
    return (int)(uint32_t)r[0];
}

}  // namespace tq2
