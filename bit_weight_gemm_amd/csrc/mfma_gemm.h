// Block-tiled MFMA product C[M][N] = f16(A[M][K]) x B[N][K]^T on gfx950,
// with B read as 2-bit ternary codes and expanded exactly to f16 in registers.
//
// Used for
//  * the ternary GEMM's large-M path ("oxibonsai-kernels 0.2.1 --
//    tests_gemm_tq2.rs": y[m][n] = sum_k x[m][k] (code-1) d): A = x staged to f16
//    (round to nearest even), B = (code-1)*d, which is exact in f16 because
//    code-1 is in {-1,0,1,2} and d is an f16 (the page's simdgroup v10 kernel
//    stages the weight tile the same way);
//  * both products of the binary low-rank forward ("cortiq-engine 0.8.43 --
//    train_mm.rs", mm_bits, which expands the sign bitmaps inside the GEMM):
//    A = f16(x.g) (staged here from f32 x and g) or f16(a.l), B = the sign
//    bitmap as the caller holds it, expanded to exact f16 +-1 in registers:
//    bits along K are read as they are (kBSign); bits along N (the contraction
//    runs down the bitmap's rows) are transposed in the LDS staging (kBSignT).
//
// Tiling: a workgroup of WM x WN x WK waves computes a BM x BN tile.  K is
// walked in steps of 64*WK*KSUB; k group wk (WM x WN waves) takes KSUB 64-wide
// slices of each step, and the groups' partial tiles are added through LDS at
// the end, in group order.  Each step the workgroup loads its A tile (f32 x
// rounded to f16, or f16 that a producer already rounded) and its B code words
// and scales, and stores them
// into STAGES XOR-swizzled LDS buffers; the waves read 16-byte A fragments and
// B code units from LDS, decode B to exact f16 in registers and issue
// v_mfma_f32_32x32x16_f16.  Loads run ahead of the LDS stores through ASTG (A)
// and BDEPTH (B) register stages.
//
// The same kernel, with other epilogues, serves the binary low-rank backward
// (the two gradient products and the recomputation of a and c); the callers are
// mfma_gemm.hip (ternary GEMM) and blr.hip (binary low-rank layer).
#pragma once

#include <hip/hip_runtime.h>

#include "bitsign.h"
#include "decode.h"
#include "internal.h"

namespace tq2 {

constexpr int BK = 64;

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Epilogues: plain f32 store; f32 store times a factor per output column;
// f16 store (round to nearest even) of the product with a factor per column,
// 0 past the first nrowf columns; f32 accumulate of the rounded product with a
// factor per column, C = f32(C + f32(f*v)) (no fused multiply-add); f32 store
// times one scalar factor alpha; both the plain f32 store (columns below nrowf)
// and the f16 store of kEpiHalfScale; the plain f32 store marked non-temporal
// (for outputs of tens of MB that this kernel never reads back: they then take
// less of the caches that the A and B tiles stream through).
enum Epi { kEpiStore = 0, kEpiRowScale = 1, kEpiHalfScale = 2, kEpiRowScaleAcc = 3, kEpiScale = 4, kEpiStoreHalf = 5,
           kEpiStoreNT = 6 };

// B operand: kBCodes, 2-bit ternary codes in the device weight layout (with
// optional scales); kBSign, a sign bitmap bits[n][ldb] with bit k%32 of word k/32
// for element (n, k), set = +1; kBSignT, a sign bitmap bits[k][ldb] with bit n%32
// of word n/32 for element (n, k) (the contraction runs down its rows).  The sign
// modes need the A operand's k order permuted within groups (perm32 for kBSign,
// perm4 for kBSignT, see bitsign.h): each A producer writes that order.
enum BMode { kBCodes = 0, kBSign = 1, kBSignT = 2 };

struct GemmArgs {
    const float *A;          // [M][lda] f32 (kAHalf: f16, read through Ah)
    const _Float16 *Ah;      // [M][lda] f16 (kAHalf)
    int64_t lda;
    const uint32_t *codes;   // [Npad][kw] code words of B (kBCodes)
    int64_t kw;
    const uint32_t *bits;    // sign bitmap (kBSign: [nbits][ldb]; kBSignT: [kbits][ldb])
    int64_t ldb;             // its words per row
    int nbits, kbits;        // the bitmap's N and K extents: kBSign rows (N) and words per row (K);
                             // kBSignT words per row (N) and rows (K); loads past them are clamped (the
                             // results there are never stored, or meet zeros of A)
    const float *g;          // kAXG/kAXGS: factor per k of A
    const uint16_t *scales;  // [Npad][kbw] f16 scales of B, or nullptr
    int64_t kbw;
    float *C;                // [M][ldc]
    _Float16 *Ch;            // [M][ldc] (kEpiHalfScale), [M][ldch] (kEpiStoreHalf)
    int64_t ldc, ldch;
    const float *rowf;       // [N] output factor (kEpiRowScale, kEpiHalfScale)
    int nrowf;               // factors present (kEpiHalfScale: columns past it get 0)
    float alpha;             // output factor (kEpiScale, the backward epilogues)
    const float *ea;         // backward epilogues: the elementwise operand E [M][ldea] (dy, a or x)
    int64_t ldea;
    float *part;             // backward epilogues: column partial sums [ceil(M/32)][nrowf]
    float gs;                // backward epilogues: gradient scale of the f16 output
    float *Cs;               // kEpiRowScaleSave / kEpiRowScaleAccSave: the product itself, [M][ldcs]
    int64_t ldcs;
    int M, N, K;             // true sizes; K bounds the A loads
    int Kloop;               // k range of one output tile: a multiple of the steps (codes are padded)
    int tiles_n;             // number of BN tiles along N
    int ksplit;              // workgroups per output tile along K (0 or 1: one), each taking
                             // Kloop/ksplit (a multiple of the steps); kEpiStore only
    int64_t cks;             // kEpiStore with ksplit > 1: chunk j of K stores its partial tile at C + j*cks
};

// LDS has 64 four-byte banks on gfx950: a 16-byte read serves 16 lanes per
// cycle, a 4-byte access 64 lanes.  Both swizzles below keep every such group
// on distinct banks (and also do so for a 32-bank LDS).
//
// A tile: 16-byte chunk `kc` (8 halves) of tile row `row`, NCH chunks per row.
// A fragment read has 16 lanes on 16 consecutive rows at one kc.  With 8 chunks
// (128 bytes) per row, rows r and r+1 are 32 banks apart, so the chunk
// permutation must differ between rows r and r+8 as well as within each group
// of 8 rows; with 16 or more chunks per row every row starts on bank 0 and the
// permutation must differ over 16 rows.
template <int NCH>
__device__ __forceinline__ int lds_off(int row, int kc) {
    const int g = NCH == 8 ? (row & 7) ^ ((row >> 3) & 1) : (row & 15);
    return row * (NCH * 8) + ((kc ^ g) << 3);
}
// B tile: slot of row R's 16-byte unit (its four code words of 64-wide k slice
// sl of the step).  The transposing store writes, per instruction, word g%4 of
// rows 4q+r for every slice and row quad a wave covers; the fragment read takes
// the units of 16 consecutive rows of one slice.  The row permutation within
// each group of 16 rows, XORed with 2*sl, puts both on distinct banks for every
// tile shape used (without the slice term a step of eight slices, whose slices
// lie a multiple of 1 KB apart, stored eight lanes to each bank).
__device__ __forceinline__ int b_slot(int row, int sl) { return row ^ ((row >> 2) & 15) ^ ((2 * sl) & 15); }

// AMODE: how A tiles are read.  kAExact: f32, K is a multiple of the step and
// rows past M read row M-1 (ternary GEMM).  kABuf: as kAExact, but through a
// buffer resource spanning the M rows, so loads of rows past M return zero
// without a memory request ((rows of the last tile)*lda*4 < 2^31).  kAHalf: A already
// rounded to f16, K a multiple of the step (zero-padded by the producer), rows
// past M read row M-1.  Rows past M only reach output rows that are never stored.
//
// kAHalfBuf: as kAHalf, through a buffer resource ((M + BM)*lda*2 < 2^31).
//
// kAXG: A = f16(x[m][k] * g[k]) from f32 x and g, the product rounded to f32
// and then to f16 (round to nearest even), stored in the perm4 k order of
// kBSignT; x is read through a buffer resource, so K must be a multiple of the
// step (no tail), rows 16-byte aligned and (M + BM)*lda*4 < 2^31.  kAXGS: the same
// from scalar loads with 64-bit addresses, for any K (pieces past K read as
// zero), alignment and size.
enum AMode { kAExact = 0, kABuf = 3, kAHalf = 4, kAXG = 5, kAXGS = 6, kAHalfBuf = 7 };

// Workgroup: WK groups of WM x WN waves.  Each step covers SK = 64*WK of K; wave
// group wk takes the 64-wide slice wk of every step, and the groups' partial
// tiles are added through LDS at the end (wk = 0, 1, ... in order).
//
// Epilogues kEpiHalfScaleP and kEpiStoreHalfP are kEpiHalfScale and
// kEpiStoreHalf with the f16 output written in the perm32 k order, as the A
// operand of a later kBSign product.
constexpr int kEpiHalfScaleP = 7, kEpiStoreHalfP = 8;

// Backward epilogues of the binary low-rank layer (v is the accumulated product,
// f the factor rowf[n], E the operand ea; columns n >= nrowf are padding: their
// f16 output is 0 and they have no partial sum).  Each keeps, per block of 32
// output rows, the column sum of E*w over the block's rows (w as below; each
// product rounded, then added in a fixed order) in part[row block][n]:
//   kEpiBwdC:  w = v (the c of the forward); Ch[m][perm4(n)] = f16((E*f)*gs);
//   kEpiBwdDb: w = v*alpha;                  Ch[m][perm32(n)] = f16((w*f)*gs);
//   kEpiBwdDx: w = v*alpha;                  C[m][n] = f*w;
//   kEpiBwdDxAcc: as kEpiBwdDx, C[m][n] = f32(C[m][n] + f32(f*w)).
constexpr int kEpiBwdC = 9, kEpiBwdDb = 10, kEpiBwdDx = 11, kEpiBwdDxAcc = 12;

// kEpiRowScale and kEpiRowScaleAcc that also keep the product v itself in
// Cs[m][n] (the binary low-rank forward's c, saved for the backward).
constexpr int kEpiRowScaleSave = 13, kEpiRowScaleAccSave = 14;

template <int BM, int BN, int WM, int WN, int WK, int STAGES, int BDEPTH, int AMODE, bool SCALED,
          int EPI, int ASTG, int KSUB, int BMODE>
__global__ __launch_bounds__(WM *WN *WK * 64) void mfma_gemm_kernel(GemmArgs p) {
    constexpr int NW = WM * WN;  // waves per k group
    constexpr int T = NW * WK * 64;
    constexpr int NSL = WK * KSUB;  // 64-wide k slices per step; group wk takes slices wk*KSUB ..
    constexpr int SK = BK * NSL;    // k per step
    constexpr int NCH = SK / 8;
    constexpr int NBLK = (SK + kBlock - 1) / kBlock;  // scale blocks per step
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MB = WTM / 32, NB = WTN / 32;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(STAGES >= 2, "at least two pipeline stages");
    static_assert(BDEPTH >= STAGES && BDEPTH % STAGES == 0, "B runs at least as far ahead as A");
    static_assert(ASTG >= 1 && BDEPTH % ASTG == 0, "A register stages");
    static_assert(BMODE == kBCodes || !SCALED, "sign bitmaps carry no scales");
    static_assert(BMODE != kBSignT || AMODE == kAXG || AMODE == kAXGS || AMODE == kAHalf || AMODE == kAHalfBuf,
                  "kBSignT needs A in the perm4 k order (kAXG, kAXGS, or a producer's f16)");
    // k-group sums go through the A tiles' LDS in RED_ROUNDS rounds, each taking
    // an equal share of the wave's MB x NB accumulator blocks
    constexpr int RED_ROUNDS = WK == 1 ? 1 : ((WK - 1) * BM * BN * 4 + STAGES * BM * SK * 2 - 1) / (STAGES * BM * SK * 2);
    static_assert((MB * NB) % RED_ROUNDS == 0, "k-group sums must split evenly over the rounds");

    // B in LDS, per mode.  kBCodes: [slice][row slot][4 code words].  kBSign:
    // [row][SROW words], the SK/32 bitmap words of the step (the 2-word pad keeps
    // the 8-byte fragment reads of 32 rows on distinct banks).  kBSignT:
    // [byte column c][k] bytes, byte c of contraction rows k (columns 8c..8c+7),
    // TSTRIDE bytes per column (the 64-byte pad keeps the 4-byte stores of 16 row
    // quads and 4 columns, and the 8-byte fragment reads, on distinct banks).
    constexpr int SW = SK / 32, SROW = SW + 2;
    constexpr int TW = BN / 32, TSTRIDE = SK + 64;
    static_assert(BMODE != kBSignT || BN % 32 == 0, "kBSignT tiles hold whole bitmap words");
    constexpr int BSM_WORDS = BMODE == kBCodes ? NSL * BN * 4 : BMODE == kBSign ? BN * SROW : (BN / 8) * TSTRIDE / 4;
    __shared__ __attribute__((aligned(16))) _Float16 As[STAGES][BM * SK];
    __shared__ __attribute__((aligned(16))) uint32_t Bsm[STAGES][BSM_WORDS];
    __shared__ __attribute__((aligned(8))) _Float16 Ds[STAGES][BMODE == kBCodes ? NBLK : 1][BN];  // B row scales

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wk = wave / NW, wr = wave % NW;
    const int wm = wr / WN, wn = wr % WN;
    const int lrow = lane & 31, hk = lane >> 5;
    const uint32_t magic = f16_magic();

    // Tile order: the hardware deals workgroups round-robin to the 8 XCDs; remap
    // so each XCD gets a contiguous run of tiles, and within the run walk N
    // first, so the workgroups sharing an A row-block share one XCD's L2.
    // With K split over workgroups, the chunks of one tile are adjacent in that
    // order, so they share an XCD too.
    const int tiles = gridDim.x;
    int tile = blockIdx.x;
    if ((tiles & 7) == 0) tile = (tile & 7) * (tiles >> 3) + (tile >> 3);
    const int ksp = EPI == kEpiStore && p.ksplit > 1 ? p.ksplit : 1;
    const int kchunk = tile % ksp;
    tile /= ksp;
    const int m0 = (tile / p.tiles_n) * BM;
    const int n0 = (tile % p.tiles_n) * BN;

    f16x acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f16x{};

    // Register stages of prefetch (see the pipeline below): STAGES for A, BDEPTH
    // for B.  Every loaded value (A as f16, B code words, bitmap words and
    // scales) goes through LDS, so a stage's registers are free again right
    // after its LDS store.  B (the weight stream) may run further ahead than A
    // (which other workgroups share through L2), to keep enough HBM reads in
    // flight when the tiles are few.
    // kBCodes: B arrives in 16-byte units holding one 16-element group of four
    // rows; a step needs BN*WK units (BN/4 row quads x 4*WK groups), BPT per
    // thread.  When there are fewer units than threads, thread t takes unit
    // t % BITEMS (duplicates load and store the same values), keeping the loop
    // free of branches; the 8-byte scale units (one row quad, one block) likewise.
    constexpr int BITEMS = BN * NSL;
    constexpr int BPT = BMODE == kBCodes ? (BITEMS + T - 1) / T : 1;
    static_assert(BMODE != kBCodes || BITEMS % T == 0 || BITEMS < T, "B units: a multiple of the threads, or fewer");
    constexpr int DITEMS = (BN / 4) * NBLK;
    static_assert(BMODE != kBCodes || (DITEMS <= T && T % DITEMS == 0), "scale units must tile the threads");
    // kBSign: one bitmap word per item (row, word of the step), SPT per thread,
    // duplicates as above.  kBSignT: thread t takes contraction row t (+T, ...) of
    // the step and loads its TW words; lanes 4q..4q+3 hold rows 4q..4q+3, which a
    // byte transpose across the quad turns into the [c][k] layout.
    constexpr int SITEMS = BN * SW;
    constexpr int SPT = BMODE == kBSign ? (SITEMS + T - 1) / T : 1;
    static_assert(BMODE != kBSign || SITEMS % T == 0 || SITEMS < T, "bitmap words: a multiple of the threads, or fewer");
    constexpr int TRPT = BMODE == kBSignT ? (SK + T - 1) / T : 1;  // contraction rows per thread
    static_assert(BMODE != kBSignT || SK % T == 0 || (SK < T && SK % 64 == 0), "bitmap rows must tile the waves");
    // A is moved in 16-byte pieces (4 floats, or 8 halves for kAHalf): piece q
    // of tile row r covers k = EPP*q .. EPP*q+EPP-1 of the step; consecutive
    // lanes take consecutive pieces of a row, so each wave-wide load reads whole
    // row segments.
    constexpr bool AXG = AMODE == kAXG || AMODE == kAXGS;
    constexpr bool AH = AMODE == kAHalf || AMODE == kAHalfBuf;
    constexpr int EPP = AH ? 8 : 4;  // elements per piece
    constexpr int QPR = SK / EPP;                  // pieces per row
    constexpr int PIECES = BM * QPR;
    constexpr int PPT = PIECES / T;
    static_assert(PIECES % T == 0, "A tile must split evenly over the threads");
    static_assert(!AXG || T % QPR == 0, "kAXG: each thread's pieces share one k range (one g load per step)");
    f4 areg[ASTG][PPT];
    f4 greg[AXG ? ASTG : 1];
    u4 breg[BMODE == kBCodes ? BDEPTH : 1][BPT];
    uint2 dreg[BMODE == kBCodes ? BDEPTH : 1];  // scales of one row quad and block
    uint32_t sreg[BMODE == kBSign ? BDEPTH : 1][SPT];
    uint32_t treg[BMODE == kBSignT ? BDEPTH : 1][TRPT][TW];

    // Buffer resources (32-bit offsets; a load past the range returns zero
    // without a memory request): A of kABuf / kAXG (f32) and kAHalfBuf (f16)
    // over its M rows, and the sign bitmap over its rows.
    const int64_t abytes = (int64_t)p.M * p.lda * (AH ? 2 : 4);
    const void *abase = AH ? static_cast<const void *>(p.Ah) : static_cast<const void *>(p.A);
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(abase), (short)0, abytes < 0x7fffffff ? (int)abytes : 0x7fffffff, 0x00020000);
    const int64_t bbytes = (int64_t)(BMODE == kBSign ? p.nbits : p.kbits) * p.ldb * 4;
    const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(p.bits), (short)0, bbytes < 0x7fffffff ? (int)bbytes : 0x7fffffff, 0x00020000);
    // element offset of each of this thread's pieces at k = 0 (gm*lda + q*EPP):
    // fixed for the whole loop, so the buffer-resource modes add k0 only
    constexpr bool ABUF = AMODE == kABuf || AMODE == kAXG || AMODE == kAHalfBuf;
    int aoff[ABUF ? PPT : 1];
    if constexpr (ABUF) {
#pragma unroll
        for (int c = 0; c < PPT; ++c) {
            const int piece = tid + c * T;
            aoff[c] = (m0 + piece / QPR) * (int)p.lda + (piece % QPR) * EPP;
        }
    }
    auto load_a = [&](int st, int k0) {
#pragma unroll
        for (int c = 0; c < PPT; ++c) {
            const int piece = tid + c * T;
            const int row = piece / QPR, q = piece % QPR;
            const int gm = m0 + row, gk = k0 + q * EPP;
            // rows past M read row M-1 (valid memory); their output rows are not stored
            const int gmc = gm < p.M ? gm : p.M - 1;
            if constexpr (AMODE == kAHalf) {
                areg[st][c] = *reinterpret_cast<const f4 *>(p.Ah + (int64_t)gmc * p.lda + gk);  // 8 halves
            } else if constexpr (AMODE == kAHalfBuf) {
                areg[st][c] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, (aoff[c] + k0) * 2, 0, 0));
            } else if constexpr (AMODE == kABuf || AMODE == kAXG) {
                areg[st][c] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, (aoff[c] + k0) * 4, 0, 0));
            } else if constexpr (AMODE == kAXGS) {
                const float *xr = p.A + (int64_t)gmc * p.lda;
#pragma unroll
                for (int e = 0; e < 4; ++e) areg[st][c][e] = gk + e < p.K ? xr[gk + e] : 0.0f;
            } else {
                static_assert(AMODE == kAExact, "A mode");
                areg[st][c] = *reinterpret_cast<const f4 *>(p.A + (int64_t)gmc * p.lda + gk);
            }
        }
        if constexpr (AXG) {  // the k range of this thread's pieces (the same for every c)
            const int gk = k0 + (tid % QPR) * EPP;
            if constexpr (AMODE == kAXG) {
                greg[st] = *reinterpret_cast<const f4 *>(p.g + gk);  // no K tail in this mode
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) greg[st][e] = gk + e < p.K ? p.g[gk + e] : 0.0f;
            }
        }
    };
    // word offset of each bitmap item at k = 0 (kBSign: row (n0 + row), word w)
    int soff[SPT];
    if constexpr (BMODE == kBSign) {
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int item = (tid + i * T) % SITEMS;
            soff[i] = (n0 + item / SW) * (int)p.ldb + item % SW;
        }
    }
    auto load_b = [&](int st, int k0) {
        if constexpr (BMODE == kBCodes) {
            const u4 *c4 = reinterpret_cast<const u4 *>(p.codes);
#pragma unroll
            for (int i = 0; i < BPT; ++i) {
                const int item = (tid + i * T) % BITEMS;
                const int64_t quad = (n0 >> 2) + item / (4 * NSL);
                breg[st][i] = c4[quad * p.kw + (k0 >> 4) + item % (4 * NSL)];
            }
            // whole waves past DITEMS skip the scales (a wave-uniform branch)
            if (SCALED && (DITEMS % 64 != 0 || tid < DITEMS)) {
                const uint2 *s4 = reinterpret_cast<const uint2 *>(p.scales);
                const int unit = tid % DITEMS, quad = unit % (BN / 4), blk = unit / (BN / 4);
                dreg[st] = s4[((n0 >> 2) + quad) * p.kbw + k0 / kBlock + blk];
            }
        } else if constexpr (BMODE == kBSign) {
            // rows past N read zero (the buffer's range); words past the row's
            // valid ones read the next row (finite signs that meet zeros of A)
#pragma unroll
            for (int i = 0; i < SPT; ++i) sreg[st][i] = __builtin_amdgcn_raw_buffer_load_b32(brsrc, (soff[i] + (k0 >> 5)) * 4, 0, 0);
        } else {
            // contraction rows past K read zero (they meet zeros of A); words past
            // the row's valid ones read the next row (columns whose results are
            // never stored, or are scaled by zero)
            if (SK >= T || tid < SK) {  // wave-uniform
#pragma unroll
                for (int rr = 0; rr < TRPT; ++rr) {
                    const int k = k0 + tid + rr * T;
                    // one base offset plus 4w: the compiler merges the TW adjacent
                    // words into 16-byte loads (a lane per contraction row, so each
                    // load instruction touches one cache line per lane)
                    const int off = (k * (int)p.ldb + (n0 >> 5)) * 4;
#pragma unroll
                    for (int w = 0; w < TW; ++w) treg[st][rr][w] = __builtin_amdgcn_raw_buffer_load_b32(brsrc, off + 4 * w, 0, 0);
                }
            }
        }
    };
    // store(st, sa, sb): A register stage sa and B register stage sb into LDS buffer st
    auto store = [&](int st, int sa, int sb) {
#pragma unroll
        for (int c = 0; c < PPT; ++c) {
            const int piece = tid + c * T;
            const int row = piece / QPR, q = piece % QPR;
            if constexpr (AH) {
                *reinterpret_cast<f4 *>(&As[st][lds_off<NCH>(row, q)]) = areg[sa][c];  // a whole 16-byte chunk
            } else {
                typedef _Float16 h4 __attribute__((ext_vector_type(4)));
                h4 v;
                if constexpr (AXG) {
                    // f16(x*g): the product rounded to f32, then to f16; stored in
                    // the perm4 order (k0, k2, k1, k3) that kBSignT's decode expects
                    const f4 xg = areg[sa][c] * greg[sa];
                    v = h4{(_Float16)xg[0], (_Float16)xg[2], (_Float16)xg[1], (_Float16)xg[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (_Float16)areg[sa][c][e];
                }
                *reinterpret_cast<h4 *>(&As[st][lds_off<NCH>(row, q >> 1) + ((q & 1) << 2)]) = v;
            }
        }
        if constexpr (BMODE == kBCodes) {
#pragma unroll
            for (int i = 0; i < BPT; ++i) {
                const int item = (tid + i * T) % BITEMS;
                const int r0 = (item / (4 * NSL)) * 4, g = item % (4 * NSL);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Bsm[st][(g >> 2) * (BN * 4) + b_slot(r0 + r, g >> 2) * 4 + (g & 3)] = breg[sb][i][r];
            }
            if (SCALED && (DITEMS % 64 != 0 || tid < DITEMS)) {
                const int unit = tid % DITEMS, quad = unit % (BN / 4), blk = unit / (BN / 4);
                *reinterpret_cast<uint2 *>(&Ds[st][blk][4 * quad]) = dreg[sb];
            }
        } else if constexpr (BMODE == kBSign) {
#pragma unroll
            for (int i = 0; i < SPT; ++i) {
                const int item = (tid + i * T) % SITEMS;
                Bsm[st][(item / SW) * SROW + item % SW] = sreg[sb][i];
            }
        } else {
            // 4x4 byte transpose across each lane quad (rows 4q..4q+3 of the step,
            // byte columns 4w..4w+3 of word w): two exchanges, with the partner
            // two lanes away and then one lane away, each keeping half the bytes
            // and taking the other half from the partner.  Lane i of the quad
            // ends with byte column 4w+i of the four rows, one row per byte.
            if (SK >= T || tid < SK) {
                const int i = lane & 3;
                const uint32_t sel2 = (i & 2) ? 0x03020706u : 0x05040100u;  // keep bytes 0,1 / take 2,3 (or the reverse)
                const uint32_t sel1 = (i & 1) ? 0x03070105u : 0x06020400u;  // keep bytes 0,2 / take 1,3 (or the reverse)
#pragma unroll
                for (int rr = 0; rr < TRPT; ++rr) {
                    const int k = tid + rr * T;  // contraction row of the step
#pragma unroll
                    for (int w = 0; w < TW; ++w) {
                        const uint32_t b = treg[sb][rr][w];
                        const uint32_t p2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x4E, 0xF, 0xF, false);  // lane ^ 2
                        const uint32_t b2 = __builtin_amdgcn_perm(p2, b, sel2);
                        const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)b2, 0xB1, 0xF, 0xF, false);  // lane ^ 1
                        const uint32_t col = __builtin_amdgcn_perm(p1, b2, sel1);
                        *reinterpret_cast<uint32_t *>(reinterpret_cast<unsigned char *>(&Bsm[st][0]) +
                                                      (4 * w + i) * TSTRIDE + (k & ~3)) = col;
                    }
                }
            }
        }
    };

    // compute(st, hook): the MFMAs of this wave's KSUB 64-wide slices of the step
    // in LDS buffer st; hook() runs after the first 16-wide sub-step, so the
    // staging of the next step overlaps the remaining MFMAs of this one.
    auto compute = [&](int st, auto &&hook) {
#pragma unroll
        for (int ks = 0; ks < KSUB; ++ks) {
            const int sl = wk * KSUB + ks;  // this wave's slice of the step
            u4 bw[NB];
            uint2 sw2[NB];
            _Float16 dv[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = wn * WTN + nb * 32 + lrow;
                if constexpr (BMODE == kBCodes) {
                    bw[nb] = *reinterpret_cast<const u4 *>(&Bsm[st][sl * (BN * 4) + b_slot(row, sl) * 4]);
                    dv[nb] = SCALED ? Ds[st][(sl * BK) / kBlock][row] : (_Float16)1.0f;
                } else if constexpr (BMODE == kBSign) {
                    sw2[nb] = *reinterpret_cast<const uint2 *>(&Bsm[st][row * SROW + 2 * sl]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h8 a[MB], b[NB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int row = wm * WTM + mb * 32 + lrow;
                    a[mb] = *reinterpret_cast<const h8 *>(&As[st][lds_off<NCH>(row, sl * 8 + 2 * j + hk)]);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if constexpr (BMODE == kBCodes) {
                        b[nb] = half_group_m1(bw[nb][j], hk, magic);
                        if constexpr (SCALED) b[nb] = b[nb] * dv[nb];
                    } else if constexpr (BMODE == kBSign) {
                        // octet 2*(j&1)+hk of the slice's word j/2 (k order perm32)
                        b[nb] = sign_octet(j < 2 ? sw2[nb].x : sw2[nb].y, 2 * (j & 1) + hk);
                    } else {
                        // column n, contraction rows sl*64 + 16j + 8hk .. +7 (k order perm4)
                        const int n = wn * WTN + nb * 32 + lrow;
                        const uint2 v = *reinterpret_cast<const uint2 *>(
                            reinterpret_cast<const unsigned char *>(&Bsm[st][0]) + (n >> 3) * TSTRIDE +
                            sl * 64 + 16 * j + 8 * hk);
                        b[nb] = sign_rows8(v.x, v.y, n & 7);
                    }
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
                if (ks == 0 && j == 0) hook();
            }
        }
    };

    // Pipeline: register stages hold steps loaded from memory but not yet in LDS;
    // LDS buffer t % STAGES holds step t.  While step t computes, step t+1 moves
    // from registers to LDS, and its register stages are refilled: A's with step
    // t+1+ASTG, B's with step t+1+BDEPTH (loads issued ASTG, or BDEPTH, steps
    // before they are stored).  One barrier per step makes step t+1's tile
    // visible; buffer (t+1) % STAGES was last read by step t+1-STAGES <= t-1,
    // which every wave finished before the barrier that ended step t-1.  The
    // step count is a multiple of BDEPTH, so the loop is branch-free; loads and
    // stores past the end use clamped addresses and are never read.
    const int nsteps = p.Kloop / (SK * ksp);
    const int kbeg = kchunk * nsteps * SK;  // this workgroup's chunk of K
    auto clampk = [&](int t) { return kbeg + (t < nsteps ? t : nsteps - 1) * SK; };
#pragma unroll
    for (int st = 0; st < BDEPTH; ++st) {
        if (st < ASTG) load_a(st, clampk(st));
        load_b(st, clampk(st));
        __builtin_amdgcn_sched_barrier(0);
    }
    store(0, 0, 0);
    load_a(0, clampk(ASTG));
    load_b(0, clampk(BDEPTH));
    __syncthreads();
    for (int t0 = 0; t0 < nsteps; t0 += BDEPTH) {
#pragma unroll
        for (int s = 0; s < BDEPTH; ++s) {
            const int t = t0 + s;
            const int nbuf = (s + 1) % STAGES;  // LDS buffer and A register stage of step t+1
            const int nsb = (s + 1) % BDEPTH;  // B register stage of step t+1
            compute(s % STAGES, [&] {
                const int nsa = (s + 1) % ASTG;  // A register stage of step t+1
                store(nbuf, nsa, nsb);
                load_a(nsa, clampk(t + 1 + ASTG));
                load_b(nsb, clampk(t + 1 + BDEPTH));
            });
            __syncthreads();
        }
    }

    // Two k groups with an even share of blocks per round split the sums: each
    // group owns half the accumulator blocks, hands the other half to its partner
    // through LDS, adds what it receives and stores its own half, so both groups
    // add and store.  Floating-point addition is commutative, so group 1's
    // acc1 + acc0 has the bits of acc0 + acc1.
    constexpr bool SPLIT = WK == 2 && (MB * NB) % (2 * RED_ROUNDS) == 0;
    constexpr int HALF = MB * NB / 2;
    // Otherwise, for the forward epilogues of four or more groups (with two, the
    // extra LDS round of group 0 costs more than the sharing saves: the split BLR
    // first product 26.5 -> 26.7 us per layer), with all the groups' tiles fitting
    // in LDS at once: every group leaves its whole partial tile there, then group g
    // adds registers g*RPG .. g*RPG+RPG-1 of every block over the groups in group
    // order (the order of group 0 adding the others, so the same bits) and stores
    // those outputs itself, so the sums and the stores are shared by all waves.
    constexpr bool BWDE = EPI == kEpiBwdC || EPI == kEpiBwdDb || EPI == kEpiBwdDx || EPI == kEpiBwdDxAcc;
    constexpr bool DIST = !SPLIT && WK >= 4 && 16 % WK == 0 && !BWDE &&
                          WK * NW * MB * NB * 1024 * 4 <= STAGES * BM * SK * 2;
    constexpr int RPG = DIST ? 16 / WK : 16;  // accumulator registers each group finishes
    if constexpr (SPLIT) {
        constexpr int HPR = HALF / RED_ROUNDS;  // blocks each group hands over per round
        float *red = reinterpret_cast<float *>(&As[0][0]);
        auto at = [&](int g, int i, int r) { return ((g * NW + wr) * HPR + i) * 1024 + r * 64 + lane; };
#pragma unroll
        for (int ro = 0; ro < RED_ROUNDS; ++ro) {
#pragma unroll
            for (int i = 0; i < HPR; ++i) {
                const int b0 = HALF + ro * HPR + i, b1 = ro * HPR + i;  // group 0 hands over b0, group 1 b1
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (wk == 0)
                        red[at(0, i, r)] = acc[b0 / NB][b0 % NB][r];
                    else
                        red[at(1, i, r)] = acc[b1 / NB][b1 % NB][r];
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < HPR; ++i) {
                const int b0 = ro * HPR + i, b1 = HALF + ro * HPR + i;  // blocks each group owns
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (wk == 0)
                        acc[b0 / NB][b0 % NB][r] += red[at(1, i, r)];
                    else
                        acc[b1 / NB][b1 % NB][r] += red[at(0, i, r)];
                }
            }
            if (ro + 1 < RED_ROUNDS) __syncthreads();
        }
    } else if constexpr (DIST) {
        float *red = reinterpret_cast<float *>(&As[0][0]);
        auto at = [&](int g, int b, int r) { return ((g * NW + wr) * (MB * NB) + b) * 1024 + r * 64 + lane; };
#pragma unroll
        for (int b = 0; b < MB * NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[at(wk, b, r)] = acc[b / NB][b % NB][r];
        __syncthreads();
#pragma unroll
        for (int b = 0; b < MB * NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (r / RPG != wk) continue;  // wave-uniform
                float v = red[at(0, b, r)];
#pragma unroll
                for (int g = 1; g < WK; ++g) v += red[at(g, b, r)];
                acc[b / NB][b % NB][r] = v;
            }
    } else if constexpr (WK > 1) {
        // k groups 1..WK-1 leave their partial tiles in LDS (over the A tiles,
        // which the loop no longer reads); group 0 adds them in group order.
        // When they do not fit at once, accumulator blocks go in rounds.
        constexpr int BPR = MB * NB / RED_ROUNDS;  // accumulator blocks per round
        float *red = reinterpret_cast<float *>(&As[0][0]);
        auto at = [&](int g, int i, int r) { return ((g * NW + wr) * BPR + i) * 1024 + r * 64 + lane; };
#pragma unroll
        for (int ro = 0; ro < RED_ROUNDS; ++ro) {
            if (wk > 0) {
#pragma unroll
                for (int i = 0; i < BPR; ++i) {
                    const int blk = ro * BPR + i;
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[at(wk - 1, i, r)] = acc[blk / NB][blk % NB][r];
                }
            }
            __syncthreads();
            if (wk == 0) {
#pragma unroll 1
                for (int g = 1; g < WK; ++g)
#pragma unroll
                    for (int i = 0; i < BPR; ++i) {
                        const int blk = ro * BPR + i;
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[blk / NB][blk % NB][r] += red[at(g - 1, i, r)];
                    }
            }
            if (ro + 1 < RED_ROUNDS) __syncthreads();
        }
        if (wk > 0) return;
    }

    // ---- epilogue: lane holds column lrow, rows 8*(r/4) + 4*hk + r%4 of each block
    constexpr bool BWD = EPI == kEpiBwdC || EPI == kEpiBwdDb || EPI == kEpiBwdDx || EPI == kEpiBwdDxAcc;
    if constexpr (BWD) {
#pragma clang fp contract(off)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (SPLIT && ((mb * NB + nb) < HALF) != (wk == 0)) continue;  // the partner group stores it (wave-uniform)
                const int gn = n0 + wn * WTN + nb * 32 + lrow;
                const int mblk = m0 + wm * WTM + mb * 32;  // first row of this 32-row block
                const bool col = gn < p.N, real = gn < p.nrowf;
                // the operands this lane reads (E, the old C of kEpiBwdDxAcc, the
                // factor), loaded before any is used, unconditionally from clamped
                // places (column 0 for padding columns, row M-1 past M), so they
                // go out together rather than one per output
                const int gnc = real ? gn : 0;
                const float f = real ? p.rowf[gnc] : 0.0f;
                float ev[16], cv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gm = mblk + 8 * (r >> 2) + 4 * hk + (r & 3);
                    const int64_t rowc = gm < p.M ? gm : p.M - 1;
                    ev[r] = p.ea[rowc * p.ldea + gnc];
                    if constexpr (EPI == kEpiBwdDxAcc) cv[r] = p.C[rowc * p.ldc + gnc];
                }
                float psum = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gm = mblk + 8 * (r >> 2) + 4 * hk + (r & 3);
                    if (gm < p.M && col) {
                        const float v = acc[mb][nb][r];
                        const int64_t row = (int64_t)gm;
                        const float e = real ? ev[r] : 0.0f;
                        if constexpr (EPI == kEpiBwdC) {
                            psum = psum + e * v;
                            p.Ch[row * p.ldch + perm4(gn)] = (_Float16)((e * f) * p.gs);
                        } else if constexpr (EPI == kEpiBwdDb) {
                            const float w = v * p.alpha;
                            psum = psum + e * w;
                            p.Ch[row * p.ldch + perm32(gn)] = (_Float16)((w * f) * p.gs);
                        } else {
                            const float w = v * p.alpha;
                            psum = psum + e * w;
                            float *c = p.C + row * p.ldc + gn;
                            if constexpr (EPI == kEpiBwdDx) *c = f * w;
                            else *c = cv[r] + f * w;
                        }
                    }
                }
                // the block's other 16 rows are in lane ^ 32: both lanes form the
                // same sum (addition is commutative), the lower one stores it
                const float other = __shfl_xor(psum, 32);
                if (hk == 0 && real && mblk < p.M) p.part[(int64_t)(mblk >> 5) * p.nrowf + gn] = psum + other;
            }
        return;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if (SPLIT && ((mb * NB + nb) < HALF) != (wk == 0)) continue;  // the partner group stores it
            const int gn = n0 + wn * WTN + nb * 32 + lrow;
            constexpr bool PAIRS = EPI == kEpiHalfScaleP || EPI == kEpiStoreHalfP;
            // (the paired f16 stores below exchange values between lanes, so no
            // lane leaves before them; their columns are checked there)
            if (!PAIRS && gn >= p.N) continue;
            float rf = 1.0f;
            constexpr bool SAVE = EPI == kEpiRowScaleSave || EPI == kEpiRowScaleAccSave;
            constexpr bool ACC = EPI == kEpiRowScaleAcc || EPI == kEpiRowScaleAccSave;
            if constexpr (EPI == kEpiRowScale || ACC || SAVE) rf = p.rowf[gn];
            constexpr bool HALF_OUT = EPI == kEpiHalfScale || EPI == kEpiStoreHalf || EPI == kEpiHalfScaleP ||
                                      EPI == kEpiStoreHalfP;
            constexpr bool PERM_OUT = EPI == kEpiHalfScaleP || EPI == kEpiStoreHalfP;
            if constexpr (HALF_OUT) rf = gn < p.nrowf ? p.rowf[gn] : 0.0f;
            const int hn = PERM_OUT ? perm32(gn) : gn;  // column of the f16 output
            if constexpr (PAIRS) {
                // f16(rf*v) in the perm32 order, where columns n and n+16 of a row
                // are adjacent: for registers r, r+1 (rows R, R'), lanes 16..31 of
                // each 32-lane half swap their row-R value for lanes 0..15's row-R'
                // value (v_permlane16_swap), so each lane stores one 4-byte pair of
                // one row (a row's 32 outputs are 64 contiguous bytes)
                _Float16 hout[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    hout[r] = (_Float16)0.0f;
                    if (DIST && r / RPG != wk) continue;  // another group stores it
                    const int gm = m0 + wm * WTM + mb * 32 + 8 * (r >> 2) + 4 * hk + (r & 3);
                    const float v = acc[mb][nb][r];
                    if constexpr (EPI == kEpiStoreHalfP)
                        if (gm < p.M && gn < p.nrowf) p.C[(int64_t)gm * p.ldc + gn] = v;
                    hout[r] = (_Float16)(rf * v);
                }
                const int cb = (gn & ~31) + (lrow & 15);  // the pair's first column
                const bool upper = (lrow & 16) != 0;
                const int64_t ldh = EPI == kEpiStoreHalfP ? p.ldch : p.ldc;
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    if (DIST && r / RPG != wk) continue;  // wave-uniform (RPG is even)
                    const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint16_t, hout[r]),
                                                                     __builtin_bit_cast(uint16_t, hout[r + 1]), false, false);
                    // lanes 0..15: row R, columns cb and cb+16; lanes 16..31: row R', the same columns
                    const int rr = upper ? r + 1 : r;
                    const int gm = m0 + wm * WTM + mb * 32 + 8 * (rr >> 2) + 4 * hk + (rr & 3);
                    if (gm < p.M && cb + 16 < p.N)
                        *reinterpret_cast<uint32_t *>(&p.Ch[(int64_t)gm * ldh + perm32(cb)]) =
                            (uint32_t)sw[0] | ((uint32_t)sw[1] << 16);
                }
                continue;
            }
            if constexpr (EPI == kEpiScale) rf = p.alpha;
            float *C = p.C + (EPI == kEpiStore ? kchunk * p.cks : 0);
            // accumulating epilogues: the old values of this lane's outputs, loaded
            // together before any is written (rows past M read row M-1)
            float cprev[16];
            if constexpr (ACC) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if (DIST && r / RPG != wk) continue;  // another group stores it
                    const int gm = m0 + wm * WTM + mb * 32 + 8 * (r >> 2) + 4 * hk + (r & 3);
                    cprev[r] = C[(int64_t)(gm < p.M ? gm : p.M - 1) * p.ldc + gn];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (DIST && r / RPG != wk) continue;  // another group stores it
                const int gm = m0 + wm * WTM + mb * 32 + 8 * (r >> 2) + 4 * hk + (r & 3);
                if (gm < p.M) {
                    const float v = acc[mb][nb][r];
                    if constexpr (EPI == kEpiHalfScale || EPI == kEpiHalfScaleP) {
                        p.Ch[(int64_t)gm * p.ldc + hn] = (_Float16)(rf * v);
                    } else if constexpr (EPI == kEpiStoreHalf || EPI == kEpiStoreHalfP) {
                        if (gn < p.nrowf) C[(int64_t)gm * p.ldc + gn] = v;
                        p.Ch[(int64_t)gm * p.ldch + hn] = (_Float16)(rf * v);
                    } else if constexpr (ACC) {
                        // two roundings: the product must not be fused into the sum
#pragma clang fp contract(off)
                        const float prod = rf * v;
                        C[(int64_t)gm * p.ldc + gn] = cprev[r] + prod;
                    } else if constexpr (EPI == kEpiStoreNT) {
                        __builtin_nontemporal_store(v, &C[(int64_t)gm * p.ldc + gn]);
                    } else
                        C[(int64_t)gm * p.ldc + gn] =
                            (EPI == kEpiRowScale || EPI == kEpiRowScaleSave || EPI == kEpiScale) ? rf * v : v;
                    if constexpr (SAVE) p.Cs[(int64_t)gm * p.ldcs + gn] = v;
                }
            }
        }
}

template <int BM, int BN, int WM, int WN, int WK, int STAGES, int AMODE, bool SCALED, int EPI,
          int BDEPTH = STAGES, int ASTG = STAGES, int KSUB = 1, int BMODE = kBCodes>
inline hipError_t run_gemm(GemmArgs p, hipStream_t s) {
    p.tiles_n = (int)((p.N + BN - 1) / BN);  // kBCodes: tiles_n * BN <= Npad, so B rows stay in bounds
    const int64_t tiles_m = (p.M + BM - 1) / BM;
    const int64_t tiles = tiles_m * p.tiles_n * (EPI == kEpiStore && p.ksplit > 1 ? p.ksplit : 1);
    mfma_gemm_kernel<BM, BN, WM, WN, WK, STAGES, BDEPTH, AMODE, SCALED, EPI, ASTG, KSUB, BMODE>
        <<<dim3((unsigned)tiles), dim3(WM * WN * WK * 64), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace tq2
