// Host repack of TQ2_0_g128 blocks into the device layout (see repack.h).
#include "repack.h"

#include <string.h>

#include "layout.h"

namespace tq2 {

namespace {

// Pair-interleaved group word: element e of the 16 at bits 2*(e>>1) + 16*(e&1).
uint32_t group_word(const uint8_t *qs4) {
    uint32_t out = 0;
    for (int e = 0; e < 16; ++e) {
        const uint32_t code = (qs4[e >> 2] >> (2 * (e & 3))) & 3u;
        out |= code << (2 * (e >> 1) + 16 * (e & 1));
    }
    return out;
}

}  // namespace

RepackLayout repack_layout(int64_t N, int64_t K) {
    RepackLayout L{};
    L.N = N, L.K = K;
    L.npad = (N + kRowPad - 1) / kRowPad * kRowPad;
    L.kw = K / 16;
    L.kb = K / kBlock;
    L.codes_bytes = (size_t)L.npad * L.kw * 4;
    const size_t scale_bytes = (size_t)L.npad * L.kb * 2;
    L.scale_off = (L.codes_bytes + 255) / 256 * 256;
    L.total = L.scale_off + (scale_bytes + 255) / 256 * 256;
    return L;
}

bool repack_blocks(const uint8_t *aos, const RepackLayout &L, uint8_t *out, bool *mfma_ok) {
    memset(out, 0, L.total);
    uint32_t *hc = reinterpret_cast<uint32_t *>(out);
    uint16_t *hs = reinterpret_cast<uint16_t *>(out + L.scale_off);
    bool ok3 = true;
    for (int64_t n = 0; n < L.N; ++n) {
        for (int64_t b = 0; b < L.kb; ++b) {
            const uint8_t *blk = aos + ((size_t)n * L.kb + b) * kBlockBytes;
            const uint16_t d = (uint16_t)(blk[32] | (blk[33] << 8));
            if (((d >> 10) & 31) == 31) return false;  // NaN or infinite scale
            bool has3 = false;
            for (int g = 0; g < 8; ++g) {
                const uint32_t wv = group_word(blk + 4 * g);
                has3 |= ((wv & (wv >> 1)) & 0x55555555u) != 0;
                hc[code_index(n, b * 8 + g, L.kw)] = wv;
            }
            // |2d| must stay within f16 for the MFMA operand (code 3 = +2d).
            if (has3 && (d & 0x7fff) > 0x77ff) ok3 = false;
            hs[scale_index(n, b, L.kb)] = d;
        }
    }
    for (int64_t n = L.N; n < L.npad; ++n)
        for (int64_t g = 0; g < L.kw; ++g) hc[code_index(n, g, L.kw)] = 0x55555555u;  // code 1 = weight 0
    if (mfma_ok) *mfma_ok = ok3;
    return true;
}

}  // namespace tq2
