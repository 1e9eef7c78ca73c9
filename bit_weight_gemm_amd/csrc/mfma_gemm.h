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
//    train_mm.rs", mm_bits): A = f16(x.g) or f16(a.l), B = the sign bitmap
//    re-laid as codes 0/2 (= -1/+1), no scale.
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

struct GemmArgs {
    const float *A;          // [M][lda] f32 (kAHalf: f16, read through Ah)
    const _Float16 *Ah;      // [M][lda] f16 (kAHalf)
    int64_t lda;
    const uint32_t *codes;   // [Npad][kw] code words of B
    int64_t kw;
    const uint16_t *scales;  // [Npad][kbw] f16 scales of B, or nullptr
    int64_t kbw;
    float *C;                // [M][ldc]
    _Float16 *Ch;            // [M][ldc] (kEpiHalfScale), [M][ldch] (kEpiStoreHalf)
    int64_t ldc, ldch;
    const float *rowf;       // [N] output factor (kEpiRowScale, kEpiHalfScale)
    int nrowf;               // factors present (kEpiHalfScale: columns past it get 0)
    float alpha;             // output factor (kEpiScale)
    int M, N, K;             // true sizes; K bounds the A loads
    int Kloop;               // k range of one workgroup: a multiple of the steps (codes are padded)
    int tiles_n;             // number of BN tiles along N
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
// B tile: slot of row R's 16-byte unit (its four code words of a 64-wide k
// slice).  The transposing store writes word g of rows 4q+r from lane 4q+g, the
// fragment read takes the units of 16 consecutive rows; this permutation within
// each group of 16 rows spreads both over all banks.
__device__ __forceinline__ int b_slot(int row) { return row ^ ((row >> 2) & 15); }

// AMODE: how A tiles are read.  kAExact: f32, K is a multiple of the step and
// rows past M read row M-1 (ternary GEMM).  kABuf: as kAExact, but through a
// buffer resource spanning the M rows, so loads of rows past M return zero
// without a memory request ((rows of the last tile)*lda*4 < 2^31).  kAHalf: A already
// rounded to f16, K a multiple of the step (zero-padded by the producer), rows
// past M read row M-1.  Rows past M only reach output rows that are never stored.
enum AMode { kAExact = 0, kABuf = 3, kAHalf = 4 };

// Workgroup: WK groups of WM x WN waves.  Each step covers SK = 64*WK of K; wave
// group wk takes the 64-wide slice wk of every step, and the groups' partial
// tiles are added through LDS at the end (wk = 0, 1, ... in order).
template <int BM, int BN, int WM, int WN, int WK, int STAGES, int BDEPTH, int AMODE, bool SCALED,
          int EPI, int ASTG, int KSUB>
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
    static_assert(ASTG >= 1 && ASTG <= STAGES && BDEPTH % ASTG == 0, "A register stages");
    // k-group sums go through the A tiles' LDS in RED_ROUNDS rounds, each taking
    // an equal share of the wave's MB x NB accumulator blocks
    constexpr int RED_ROUNDS = WK == 1 ? 1 : ((WK - 1) * BM * BN * 4 + STAGES * BM * SK * 2 - 1) / (STAGES * BM * SK * 2);
    static_assert((MB * NB) % RED_ROUNDS == 0, "k-group sums must split evenly over the rounds");

    __shared__ __attribute__((aligned(16))) _Float16 As[STAGES][BM * SK];
    __shared__ __attribute__((aligned(16))) uint32_t Bs[STAGES][NSL][BN * 4];  // 4 code words per row and slice
    __shared__ __attribute__((aligned(8))) _Float16 Ds[STAGES][NBLK][BN];     // B row scales of the step

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wk = wave / NW, wr = wave % NW;
    const int wm = wr / WN, wn = wr % WN;
    const int lrow = lane & 31, hk = lane >> 5;
    const uint32_t magic = f16_magic();

    // Tile order: the hardware deals workgroups round-robin to the 8 XCDs; remap
    // so each XCD gets a contiguous run of tiles, and within the run walk N
    // first, so the workgroups sharing an A row-block share one XCD's L2.
    const int tiles = gridDim.x;
    int tile = blockIdx.x;
    if ((tiles & 7) == 0) tile = (tile & 7) * (tiles >> 3) + (tile >> 3);
    const int m0 = (tile / p.tiles_n) * BM;
    const int n0 = (tile % p.tiles_n) * BN;

    f16x acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f16x{};

    // Register stages of prefetch (see the pipeline below): STAGES for A, BDEPTH
    // for B.  Every loaded value (A as f16, B code words and scales) goes through
    // LDS, so a stage's registers are free again right after its LDS store.  B
    // (the weight stream) may run further ahead than A (which other workgroups
    // share through L2), to keep enough HBM reads in flight when the tiles are
    // few.
    // B arrives in 16-byte units holding one 16-element group of four rows; a
    // step needs BN*WK units (BN/4 row quads x 4*WK groups), BPT per thread.
    // When there are fewer units than threads, thread t takes unit t % BITEMS
    // (duplicates load and store the same values), keeping the loop free of
    // branches; the 8-byte scale units (one row quad, one block) likewise.
    constexpr int BITEMS = BN * NSL;
    constexpr int BPT = (BITEMS + T - 1) / T;
    static_assert(BITEMS % T == 0 || BITEMS < T, "B units: a multiple of the threads, or fewer");
    constexpr int DITEMS = (BN / 4) * NBLK;
    static_assert(DITEMS <= T && T % DITEMS == 0, "scale units must tile the threads");
    // A is moved in 16-byte pieces (4 floats, or 8 halves for kAHalf): piece q
    // of tile row r covers k = EPP*q .. EPP*q+EPP-1 of the step; consecutive
    // lanes take consecutive pieces of a row, so each wave-wide load reads whole
    // row segments.
    constexpr int EPP = AMODE == kAHalf ? 8 : 4;  // elements per piece
    constexpr int QPR = SK / EPP;                  // pieces per row
    constexpr int PIECES = BM * QPR;
    constexpr int PPT = PIECES / T;
    static_assert(PIECES % T == 0, "A tile must split evenly over the threads");
    f4 areg[ASTG][PPT];
    u4 breg[BDEPTH][BPT];
    uint2 dreg[BDEPTH];  // scales of one row quad and block

    // (only kABuf reads through it; unused otherwise)
    const int64_t abytes = (int64_t)p.M * p.lda * 4;
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(p.A), (short)0, abytes < 0x7fffffff ? (int)abytes : 0x7fffffff, 0x00020000);
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
            } else if constexpr (AMODE == kABuf) {
                areg[st][c] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(arsrc, (gm * (int)p.lda + gk) * 4, 0, 0));
            } else {
                static_assert(AMODE == kAExact, "A mode");
                areg[st][c] = *reinterpret_cast<const f4 *>(p.A + (int64_t)gmc * p.lda + gk);
            }
        }
    };
    auto load_b = [&](int st, int k0) {
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
    };
    // store(st, sa, sb): A register stage sa and B register stage sb into LDS buffer st
    auto store = [&](int st, int sa, int sb) {
#pragma unroll
        for (int c = 0; c < PPT; ++c) {
            const int piece = tid + c * T;
            const int row = piece / QPR, q = piece % QPR;
            if constexpr (AMODE == kAHalf) {
                *reinterpret_cast<f4 *>(&As[st][lds_off<NCH>(row, q)]) = areg[sa][c];  // a whole 16-byte chunk
            } else {
                typedef _Float16 h4 __attribute__((ext_vector_type(4)));
                h4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (_Float16)areg[sa][c][e];
                *reinterpret_cast<h4 *>(&As[st][lds_off<NCH>(row, q >> 1) + ((q & 1) << 2)]) = v;
            }
        }
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int item = (tid + i * T) % BITEMS;
            const int r0 = (item / (4 * NSL)) * 4, g = item % (4 * NSL);
#pragma unroll
            for (int r = 0; r < 4; ++r) Bs[st][g >> 2][b_slot(r0 + r) * 4 + (g & 3)] = breg[sb][i][r];
        }
        if (SCALED && (DITEMS % 64 != 0 || tid < DITEMS)) {
            const int unit = tid % DITEMS, quad = unit % (BN / 4), blk = unit / (BN / 4);
            *reinterpret_cast<uint2 *>(&Ds[st][blk][4 * quad]) = dreg[sb];
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
            _Float16 dv[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = wn * WTN + nb * 32 + lrow;
                bw[nb] = *reinterpret_cast<const u4 *>(&Bs[st][sl][b_slot(row) * 4]);
                dv[nb] = SCALED ? Ds[st][(sl * BK) / kBlock][row] : (_Float16)1.0f;
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
                    b[nb] = half_group_m1(bw[nb][j], hk, magic);
                    if constexpr (SCALED) b[nb] = b[nb] * dv[nb];
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
    const int nsteps = p.Kloop / SK;
    auto clampk = [&](int t) { return (t < nsteps ? t : nsteps - 1) * SK; };
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
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if (SPLIT && ((mb * NB + nb) < HALF) != (wk == 0)) continue;  // the partner group stores it
            const int gn = n0 + wn * WTN + nb * 32 + lrow;
            if (gn >= p.N) continue;
            float rf = 1.0f;
            if constexpr (EPI == kEpiRowScale || EPI == kEpiRowScaleAcc) rf = p.rowf[gn];
            if constexpr (EPI == kEpiHalfScale || EPI == kEpiStoreHalf) rf = gn < p.nrowf ? p.rowf[gn] : 0.0f;
            if constexpr (EPI == kEpiScale) rf = p.alpha;
            float *C = p.C;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm * WTM + mb * 32 + 8 * (r >> 2) + 4 * hk + (r & 3);
                if (gm < p.M) {
                    const float v = acc[mb][nb][r];
                    if constexpr (EPI == kEpiHalfScale) {
                        p.Ch[(int64_t)gm * p.ldc + gn] = (_Float16)(rf * v);
                    } else if constexpr (EPI == kEpiStoreHalf) {
                        if (gn < p.nrowf) C[(int64_t)gm * p.ldc + gn] = v;
                        p.Ch[(int64_t)gm * p.ldch + gn] = (_Float16)(rf * v);
                    } else if constexpr (EPI == kEpiRowScaleAcc) {
                        // two roundings: the product must not be fused into the sum
#pragma clang fp contract(off)
                        float *c = C + (int64_t)gm * p.ldc + gn;
                        const float prod = rf * v;
                        *c = *c + prod;
                    } else if constexpr (EPI == kEpiStoreNT) {
                        __builtin_nontemporal_store(v, &C[(int64_t)gm * p.ldc + gn]);
                    } else
                        C[(int64_t)gm * p.ldc + gn] = (EPI == kEpiRowScale || EPI == kEpiScale) ? rf * v : v;
                }
            }
        }
}

template <int BM, int BN, int WM, int WN, int WK, int STAGES, int AMODE, bool SCALED, int EPI,
          int BDEPTH = STAGES, int ASTG = STAGES, int KSUB = 1>
inline hipError_t run_gemm(GemmArgs p, hipStream_t s) {
    p.tiles_n = (int)((p.N + BN - 1) / BN);  // tiles_n * BN <= Npad, so B rows stay in bounds
    const int64_t tiles_m = (p.M + BM - 1) / BM;
    const int64_t tiles = tiles_m * p.tiles_n;
    mfma_gemm_kernel<BM, BN, WM, WN, WK, STAGES, BDEPTH, AMODE, SCALED, EPI, ASTG, KSUB>
        <<<dim3((unsigned)tiles), dim3(WM * WN * WK * 64), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace tq2
