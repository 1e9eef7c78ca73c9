// Host check of the weight repack (csrc/repack.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer: random blocks of every code and of finite f16
// scales (subnormal and negative included) are repacked into exactly sized
// buffers and read back through the layout's index functions, element by
// element, against the block format; padding rows, the non-finite scale
// refusal and the f16-range flag of the MFMA operand are checked too.  Built and
// run by tests/test_sanitize_host.py with g++.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../bit_weight_gemm_amd/csrc/layout.h"
#include "../../bit_weight_gemm_amd/csrc/repack.h"

static int fails = 0;
#define CHECK(c, msg) do { if (!(c)) { fprintf(stderr, "FAIL: %s\n", msg); ++fails; } } while (0)

static uint32_t rng = 0x9E3779B1u;
static uint32_t next() { rng ^= rng << 13; rng ^= rng >> 17; rng ^= rng << 5; return rng; }

static uint16_t finite_half() {
    for (;;) {
        uint16_t h = (uint16_t)next();
        if (((h >> 10) & 31) != 31 && (h & 0x7fff) <= 0x77ff) return h;  // |2d| stays finite
    }
}

static void round_trip(int64_t N, int64_t K) {
    const int64_t kb = K / 128;
    std::vector<uint8_t> aos((size_t)N * kb * 34);
    for (size_t i = 0; i < aos.size(); i += 34) {
        for (int j = 0; j < 32; ++j) aos[i + j] = (uint8_t)next();
        const uint16_t d = finite_half();
        aos[i + 32] = (uint8_t)(d & 255), aos[i + 33] = (uint8_t)(d >> 8);
    }
    const tq2::RepackLayout L = tq2::repack_layout(N, K);
    CHECK(L.npad % tq2::kRowPad == 0 && L.npad >= N && L.npad - N < tq2::kRowPad, "row padding");
    uint8_t *out = (uint8_t *)malloc(L.total);  // exactly the image size
    bool ok3 = false;
    CHECK(tq2::repack_blocks(aos.data(), L, out, &ok3), "finite scales accepted");
    CHECK(ok3, "scales within half of f16 range: MFMA operand allowed");
    const uint32_t *codes = (const uint32_t *)out;
    const uint16_t *scales = (const uint16_t *)(out + L.scale_off);
    for (int64_t n = 0; n < L.npad; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const uint32_t w = codes[tq2::code_index(n, k / 16, L.kw)];
            const int e = (int)(k % 16);
            const int code = (int)((w >> (2 * (e >> 1) + 16 * (e & 1))) & 3u);
            const uint16_t d = scales[tq2::scale_index(n, k / 128, L.kb)];
            if (n < N) {
                const uint8_t *blk = &aos[((size_t)n * kb + k / 128) * 34];
                const int want = (blk[(k % 128) / 4] >> (2 * (k % 4))) & 3;
                CHECK(code == want, "code of (n, k)");
                CHECK(d == (uint16_t)(blk[32] | (blk[33] << 8)), "scale of (n, block)");
            } else {
                CHECK(code == 1 && d == 0, "padding rows: code 1, scale 0");
            }
        }
    free(out);
}

int main() {
    const int64_t shapes[][2] = {{1, 128}, {40, 256}, {257, 384}, {4, 4096}};
    for (auto &s : shapes) round_trip(s[0], s[1]);
    // a NaN or infinite scale is refused
    const tq2::RepackLayout L = tq2::repack_layout(2, 128);
    std::vector<uint8_t> aos(2 * 34, 0x55);
    uint8_t *out = (uint8_t *)malloc(L.total);
    for (uint16_t bad : {(uint16_t)0x7c00, (uint16_t)0xfc00, (uint16_t)0x7e01}) {
        aos[34 + 32] = (uint8_t)(bad & 255), aos[34 + 33] = (uint8_t)(bad >> 8);
        CHECK(!tq2::repack_blocks(aos.data(), L, out, nullptr), "non-finite scale refused");
    }
    // code 3 with |d| > 0x77ff: 2d overflows f16, the MFMA operand is not allowed
    aos[34 + 32] = 0x00, aos[34 + 33] = 0x78;  // d = 32768
    aos[34] = 0x03;                             // element 0 of the second row: code 3
    bool ok3 = true;
    CHECK(tq2::repack_blocks(aos.data(), L, out, &ok3) && !ok3, "code 3 with |2d| beyond f16 flagged");
    aos[34] = 0x55;                             // no code 3: the large scale is harmless
    CHECK(tq2::repack_blocks(aos.data(), L, out, &ok3) && ok3, "large scale without code 3 allowed");
    free(out);
    if (fails) return 1;
    printf("repack ok\n");
    return 0;
}
