// Device weight layout of libtq2 (built by the host repack from the
// array-of-structs blocks), usable from host-only C++ and from HIP device code
// (constexpr functions are host and device functions under HIP):
//   codes  : u32 [Npad/4][K/16][4]   one word per 16 consecutive elements of a row;
//            the words of rows 4i..4i+3 for the same 16-element group g are
//            adjacent (16 bytes), so one 16-byte load fetches a group of four rows.
//            Element e (0..15) of a group sits in bits 2*(e>>1) + 16*(e&1): even
//            elements fill the low half, odd elements the high half, each as the
//            2-bit code of the block format.  A word thus yields element pairs
//            (2s, 2s+1) as the two halves of one 32-bit register, the shape both
//            the f32 path (one pair per decode) and the MFMA operand (consecutive
//            k in the low/high halves) consume.
//   scales : u16 [Npad/4][K/128][4]  f16 bit pattern of each block's d, four rows
//            per 8-byte unit in the same row grouping.
//   Rows n >= N up to Npad (a multiple of kRowPad) hold code 1 and scale 0.
//   Word (n, g) lives at codes[((n/4) * (K/16) + g) * 4 + n%4]; scale (n, b) at
//   scales[((n/4) * (K/128) + b) * 4 + n%4].
#pragma once

#include <stdint.h>

namespace tq2 {

constexpr int kBlock = 128;      // weights per block
constexpr int kRowPad = 256;     // device rows are padded to a multiple of this

// Index of word (n, g) / scale (n, b) in the interleaved planes.
constexpr int64_t code_index(int64_t n, int64_t g, int64_t kw) { return ((n >> 2) * kw + g) * 4 + (n & 3); }
constexpr int64_t scale_index(int64_t n, int64_t b, int64_t kb) { return ((n >> 2) * kb + b) * 4 + (n & 3); }

}  // namespace tq2
