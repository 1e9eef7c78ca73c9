// The ternary GEMM's MFMA path ("oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs":
// y[m][n] = sum_k x[m][k] (code-1) d, row-major [M][N], overwritten): the tile
// configuration of the block-tiled kernel in mfma_gemm.h for each range of M.
#include <atomic>

#include "mfma_gemm.h"

namespace tq2 {

static int mfma_stages(int64_t K) { return (K / BK) % 4 == 0 ? 4 : 2; }

// Compute units of the current device, cached per device ordinal.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load();
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev < 64) cache[dev].store(cus);
    return cus;
}

// Large-M tile height: every workgroup of a round runs one tile, so a launch
// takes about (rounds of workgroups) x (rows per tile) units of time.  96-row
// tiles win where 128-row tiles leave a round half empty (1536 x 3072: 144
// tiles for 256 CUs; 1536 x 27648: 1296 tiles, a sixth round of 16).
static bool rows96(int64_t M, int64_t N, int cus) {
    const int64_t tn = (N + 255) / 256;
    const int64_t r128 = ((M + 127) / 128 * tn + cus - 1) / cus;
    const int64_t r96 = ((M + 95) / 96 * tn + cus - 1) / cus;
    return r96 * 96 < r128 * 128;
}

hipError_t launch_gemm_mfma(const DevWeight &w, const float *x, float *y, int64_t M, hipStream_t s) {
    GemmArgs p{};
    p.A = x;
    p.lda = w.K;
    p.codes = w.codes;
    p.kw = w.K / 16;
    p.scales = w.scales;
    p.kbw = w.K / kBlock;
    p.C = y;
    p.ldc = w.N;
    p.rowf = nullptr;
    p.M = (int)M;
    p.N = (int)w.N;
    p.K = (int)w.K;
    p.Kloop = (int)w.K;
    // K is a multiple of 128 (two steps); four stages when the step count allows
    const bool four = mfma_stages(w.K) == 4;
    // Small M: 64-column tiles whose four waves of each column half split the
    // step's K four ways (two ways when K has too few blocks), so N/64
    // workgroups of eight waves stream the weight.  When K/128 is a multiple of
    // 8 (33 to 64 rows; up to 32 rows such K goes to the skinny kernel), each
    // wave takes two 64-wide slices of a 512-wide step: with so little MFMA
    // work per step, fewer steps (and barriers) matter most.  Up to 32 rows, A
    // comes through a buffer resource, so the rows past M cost no memory
    // traffic.
    const int64_t kb = w.K / kBlock;
    if (M <= 32 && M * w.K * 4 < ((int64_t)1 << 31)) {
        if (kb % 4 == 0) return run_gemm<32, 64, 1, 2, 4, 2, kABuf, true, kEpiStore>(p, s);
        if (kb % 2 == 0) return run_gemm<32, 64, 1, 2, 2, 2, kABuf, true, kEpiStore>(p, s);
    } else if (M <= 64) {
        if (kb % 8 == 0) return run_gemm<64, 64, 1, 2, 4, 2, kAExact, true, kEpiStore, 2, 1, 2>(p, s);
        if (kb % 4 == 0) return run_gemm<64, 64, 1, 2, 2, 4, kAExact, true, kEpiStore>(p, s);
        if (kb % 2 == 0) return run_gemm<64, 64, 1, 2, 2, 2, kAExact, true, kEpiStore>(p, s);
    }
    if (M <= 64)
        return four ? run_gemm<32, 256, 1, 4, 1, 4, kAExact, true, kEpiStore>(p, s)
                    : run_gemm<32, 256, 1, 4, 1, 2, kAExact, true, kEpiStore>(p, s);
    // Large M: 128 x 256 tiles of eight waves, two per SIMD: four column waves
    // times two k groups, each k group taking one 64-wide half of a 128-wide
    // step (two LDS buffers, one A register stage).  y (32 MB at M=2048,
    // N=4096) is stored non-temporally.  Where the tile count fills the rounds
    // of workgroups better, 96 x 256 tiles (two A register stages fit).  x is
    // read through a buffer resource (32-bit offsets: 10 fewer registers than
    // 64-bit addresses) while it and the rows of the last tile lie within 2 GB.
    if (kb % 2 == 0) {
        const bool abuf = (M + 256) * w.K * 4 < ((int64_t)1 << 31);
        if (rows96(M, w.N, device_cus()))
            return abuf ? run_gemm<96, 256, 1, 4, 2, 2, kABuf, true, kEpiStoreNT, 2, 2>(p, s)
                        : run_gemm<96, 256, 1, 4, 2, 2, kAExact, true, kEpiStoreNT, 2, 2>(p, s);
        return abuf ? run_gemm<128, 256, 1, 4, 2, 2, kABuf, true, kEpiStoreNT, 2, 1>(p, s)
                    : run_gemm<128, 256, 1, 4, 2, 2, kAExact, true, kEpiStoreNT, 2, 1>(p, s);
    }
    return four ? run_gemm<128, 256, 1, 4, 1, 4, kAExact, true, kEpiStoreNT>(p, s)
                : run_gemm<128, 256, 1, 4, 1, 2, kAExact, true, kEpiStoreNT>(p, s);
}

}  // namespace tq2
