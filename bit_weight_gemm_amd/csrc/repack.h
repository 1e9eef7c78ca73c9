// Host repack of TQ2_0_g128 weight blocks into the device layout (layout.h).
// Plain C++, no HIP: the C ABI calls it before copying the result to the GPU.
//
// Block format ("oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs", block struct and
// correctness test): 32 bytes of 2-bit codes, element e of the block at bits
// 2*(e%4) of byte e/4, then the f16 scale d, little-endian; w = (code - 1) * d.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace tq2 {

constexpr size_t kBlockBytes = 34;

// Sizes of the device image of an N x K weight (K a multiple of kBlock).
struct RepackLayout {
    int64_t N, K, npad, kw, kb;
    size_t codes_bytes;   // the code plane
    size_t scale_off;     // offset of the scale plane (256-byte aligned)
    size_t total;         // bytes of the whole image (256-byte multiple)
};
RepackLayout repack_layout(int64_t N, int64_t K);

// Writes the device image of `aos` (N*(K/128)*34 bytes) into `out` (L.total
// bytes, caller-owned, any contents).  Returns false, with `out` partly written,
// when a block's scale is NaN or infinite.  *mfma_ok is set to whether every
// block holding a code 3 (w = +2d) has |2d| within f16 range, the condition of
// the f16 MFMA operand.
bool repack_blocks(const uint8_t *aos, const RepackLayout &L, uint8_t *out, bool *mfma_ok);

}  // namespace tq2
