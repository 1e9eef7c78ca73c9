// Exact in-register decode of sign bitmaps (binary low-rank layer: a set bit is
// +1, a clear bit -1) to f16 MFMA operands on gfx950, and the k orders those
// operands come in.
#pragma once

#include "decode.h"

namespace tq2 {

// ---- sign bits (binary low-rank layer: a set bit is +1, a clear bit -1)
//
// In f16, +1 (0x3C00) and -1 (0xBC00) differ only in the sign bit.  With the
// two bits of a pair rotated to positions 15 and 31 (the halves' sign bits),
// keeping just those two bits and flipping -1 by them gives (2b - 1) in each
// half: one rotation and one three-input bitwise operation (v_bitop3_b32) per
// pair, the values exact.
__device__ __forceinline__ uint32_t sign_pair15(uint32_t t) { return (t & 0x80008000u) ^ 0xBC00BC00u; }
// `w` rotated right by `s` (mod 32)
__device__ __forceinline__ uint32_t rotr(uint32_t w, uint32_t s) { return __builtin_amdgcn_alignbit(w, w, s & 31u); }

// Octet o (0..3) of a word of 32 sign bits along k as an MFMA operand: the eight
// elements are k = 4o+i and 4o+i+16 for i = 0..3, in the order 4o, 4o+16, 4o+1,
// 4o+17, ...  Pair i (bits 4o+i and 4o+i+16) is rotated right by 4o+i-15 to the
// sign bits.  The A operand must hold the same k order (perm32 below).
__device__ __forceinline__ h8 sign_octet(uint32_t w, int o) {
    const uint32_t s = (uint32_t)(4 * o + 17);
    const h2 p0 = as_h2(sign_pair15(rotr(w, s))), p1 = as_h2(sign_pair15(rotr(w, s + 1))),
             p2 = as_h2(sign_pair15(rotr(w, s + 2))), p3 = as_h2(sign_pair15(rotr(w, s + 3)));
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Position of k within its group of 32 in that order: k = 4o+i+16h sits at 8o+2i+h.
__host__ __device__ inline int perm32(int k) {
    return (k & ~31) | (((k & 15) >> 2) << 3) | ((k & 3) << 1) | ((k >> 4) & 1);
}

// Eight sign bits of one column from eight contraction rows, as the column's byte
// (bit p) of rows k0..k3 in `lo` and k4..k7 in `hi` (row r in byte r), as an MFMA
// operand in the k order k0, k2, k1, k3, k4, k6, k5, k7: rows two apart sit 16 bits
// apart, so rotating right by p-15 puts rows k0 and k2 on the sign bits, and by
// p-7 rows k1 and k3.  The A operand must hold the same k order (perm4 below).
__device__ __forceinline__ h8 sign_rows8(uint32_t lo, uint32_t hi, int p) {
    const uint32_t s0 = (uint32_t)(p + 17), s1 = (uint32_t)(p + 25);
    const h2 p0 = as_h2(sign_pair15(rotr(lo, s0))), p1 = as_h2(sign_pair15(rotr(lo, s1))),
             p2 = as_h2(sign_pair15(rotr(hi, s0))), p3 = as_h2(sign_pair15(rotr(hi, s1)));
    return h8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Position of k within its group of 4 in that order: 0, 2, 1, 3 (its own inverse).
__host__ __device__ inline int perm4(int k) { return (k & ~3) | ((k & 1) << 1) | ((k >> 1) & 1); }

}  // namespace tq2
