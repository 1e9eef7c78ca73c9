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
// (the two gradient products and the recomputation of a and c), below the
// forward.
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
// and the f16 store of kEpiHalfScale.
enum Epi { kEpiStore = 0, kEpiRowScale = 1, kEpiHalfScale = 2, kEpiRowScaleAcc = 3, kEpiScale = 4, kEpiStoreHalf = 5 };

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
// without a memory request (small M, M*lda*4 < 2^31).  kAHalf: A already
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

    if constexpr (WK > 1) {
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
                    } else
                        C[(int64_t)gm * p.ldc + gn] = (EPI == kEpiRowScale || EPI == kEpiScale) ? rf * v : v;
                }
            }
        }
}

template <int BM, int BN, int WM, int WN, int WK, int STAGES, int AMODE, bool SCALED, int EPI,
          int BDEPTH = STAGES, int ASTG = STAGES, int KSUB = 1>
static hipError_t run_gemm(GemmArgs p, hipStream_t s) {
    p.tiles_n = (int)((p.N + BN - 1) / BN);  // tiles_n * BN <= Npad, so B rows stay in bounds
    const int64_t tiles_m = (p.M + BM - 1) / BM;
    const int64_t tiles = tiles_m * p.tiles_n;
    mfma_gemm_kernel<BM, BN, WM, WN, WK, STAGES, BDEPTH, AMODE, SCALED, EPI, ASTG, KSUB>
        <<<dim3((unsigned)tiles), dim3(WM * WN * WK * 64), 0, s>>>(p);
    return hipGetLastError();
}

// ------------------------------------------------------------------ ternary GEMM, large M

static int mfma_stages(int64_t K) { return (K / BK) % 4 == 0 ? 4 : 2; }

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
    // 8, each wave takes two 64-wide slices of a 512-wide step: with so little
    // MFMA work per step, fewer steps (and barriers) matter most.  Up to 32
    // rows, A comes through a buffer resource, so the rows past M cost no memory
    // traffic.
    const int64_t kb = w.K / kBlock;
    if (M <= 32 && M * w.K * 4 < ((int64_t)1 << 31)) {
        if (kb % 8 == 0) return run_gemm<32, 64, 1, 2, 4, 2, kABuf, true, kEpiStore, 2, 1, 2>(p, s);
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
    // step (two LDS buffers, one A register stage).
    if (kb % 2 == 0) return run_gemm<128, 256, 1, 4, 2, 2, kAExact, true, kEpiStore, 2, 1>(p, s);
    return four ? run_gemm<128, 256, 1, 4, 1, 4, kAExact, true, kEpiStore>(p, s)
                : run_gemm<128, 256, 1, 4, 1, 2, kAExact, true, kEpiStore>(p, s);
}

// ------------------------------------------------------------------ binary low-rank forward

static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Tiles of the two products.  The preparation pass re-lays both bitmaps and
// writes f16(x*g) (the A operand of GEMM1, zero-padded in K).  GEMM1 (M x r,
// K = d_in) writes f16(l * a), the A operand of GEMM2 (M x d_out, K = r), from
// its epilogue; its columns past r are zero.  Small M takes 32 x 64 tiles of
// GEMM1 (eight waves, four k groups) so that enough workgroups stream the long
// K without splitting it; larger M takes 128 x 128 tiles.
constexpr int kBlrKPad = 512;     // GEMM1's K padding: whole pipeline rounds of either tile
constexpr int kBlr2Step = 2 * 2 * BK;  // GEMM2: two k groups x 64, two stages

static bool blr_small_tiles(int64_t M, int64_t kpad2) { return ((M + 31) / 32) * (kpad2 / 64) < 2048; }

BlrPlan blr_plan(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    BlrPlan p{};
    p.M = M, p.d_in = d_in, p.d_out = d_out, p.r = r;
    p.kpad1 = round_up(d_in, kBlrKPad);
    p.kpad2 = round_up(r, kBlr2Step);
    p.npad1 = round_up(r, kRowPad);
    p.npad2 = round_up(d_out, kRowPad);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (size_t)round_up((int64_t)(off + bytes), 256);
        return at;
    };
    p.off_codes_v = take((size_t)p.npad1 * (p.kpad1 / 16) * 4);
    p.off_codes_u = take((size_t)p.npad2 * (p.kpad2 / 16) * 4);
    p.off_al = take((size_t)M * p.kpad2 * 2);
    p.off_xg = take((size_t)M * p.kpad1 * 2);
    p.total = off;
    return p;
}

// Sign bitmaps -> code words (set bit -> code 2 = +1, clear -> code 0 = -1,
// padding -> code 1 = 0) in the device layout, with row index n and
// contraction index k, for both matrices in one launch.  A thread makes the
// 16-byte unit of four rows (4q .. 4q+3) for one 16-wide k group g.
//   S_V: sign(n, k) = bit n of bits_v[k][n/32]   (n = rank, k = input j): a wave
//        takes 64 consecutive row quads of one group, so each of its 16 loads
//        (one per k) touches 8 bitmap words shared by the lanes;
//   S_U: sign(n, k) = bit k of bits_u[n][k/32]   (n = output i, k = rank): a
//        wave takes 64 consecutive groups of one row quad, so its loads read
//        whole bitmap rows and its stores are contiguous.
// Out-of-range elements read a valid word and are replaced by code 1.
// Blocks from nblk_v + nblk_u on write xg[m][k] = f16(x[m][k] * g[k]) (product in
// f32, round to nearest even) for k < d_in and 0 up to kpad1, 8 values per thread.
struct BlrPrep {
    const uint32_t *bits_v, *bits_u;
    uint32_t *codes_v, *codes_u;
    const float *x, *g;
    _Float16 *xg;
    int64_t words;                     // r / 32
    int64_t M, r, d_in, d_out;
    int64_t npad1, kpad1, npad2, kpad2;
    int64_t nblk_v, nblk_u;
    int xvec;                          // x rows and g allow 16-byte loads
};

// code of element e (0..15) at its place in a group word
__device__ __forceinline__ uint32_t code_at(uint32_t code, int e) { return code << (2 * (e >> 1) + 16 * (e & 1)); }

__global__ __launch_bounds__(256) void blr_prep_kernel(BlrPrep q) {
    const int64_t bid = blockIdx.x;
    if (bid < q.nblk_v) {
        const int64_t kw = q.kpad1 / 16, quads = q.npad1 / 4;
        const int64_t qblocks = (quads + 255) / 256;
        const int64_t quad = (bid % qblocks) * 256 + threadIdx.x, g = bid / qblocks;
        if (quad >= quads) return;
        const int64_t n0 = quad * 4;
        const bool nin = n0 < q.r;  // r % 32 == 0: a quad is wholly inside or wholly past r
        const int64_t wrd = nin ? n0 >> 5 : 0;
        const int sh = (int)(n0 & 31);
        u4 out = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t k = g * 16 + e;
            const bool in = nin && k < q.d_in;
            const uint32_t bits = (q.bits_v[(in ? k : 0) * q.words + wrd] >> sh) & 15u;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                out[rr] |= code_at(in ? (((bits >> rr) & 1u) ? 2u : 0u) : 1u, e);
        }
        *reinterpret_cast<u4 *>(q.codes_v + (quad * kw + g) * 4) = out;
    } else if (bid < q.nblk_v + q.nblk_u) {
        const int64_t kw = q.kpad2 / 16;
        const int64_t gblocks = (kw + 255) / 256;
        const int64_t rel = bid - q.nblk_v;
        const int64_t quad = rel / gblocks, g = (rel % gblocks) * 256 + threadIdx.x;
        if (g >= kw) return;
        u4 out;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t n = quad * 4 + rr;
            const bool in = n < q.d_out && g * 16 < q.r;
            const uint32_t half = (q.bits_u[(in ? n : 0) * q.words + (in ? g >> 1 : 0)] >> (16 * (g & 1))) & 0xFFFFu;
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const bool ine = in && g * 16 + e < q.r;
                w |= code_at(ine ? (((half >> e) & 1u) ? 2u : 0u) : 1u, e);
            }
            out[rr] = w;
        }
        *reinterpret_cast<u4 *>(q.codes_u + (quad * kw + g) * 4) = out;
    } else {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        const int64_t per_row = q.kpad1 / 8;
        const int64_t piece = (bid - q.nblk_v - q.nblk_u) * 256 + threadIdx.x;
        if (piece >= q.M * per_row) return;
        const int64_t m = piece / per_row, k0 = (piece % per_row) * 8;
        const float *xr = q.x + m * q.d_in;
        h8 out;
        if (q.xvec && k0 + 8 <= q.d_in) {
            const f4 x0 = *reinterpret_cast<const f4 *>(xr + k0), x1 = *reinterpret_cast<const f4 *>(xr + k0 + 4);
            const f4 g0 = *reinterpret_cast<const f4 *>(q.g + k0), g1 = *reinterpret_cast<const f4 *>(q.g + k0 + 4);
            const f4 p0 = x0 * g0, p1 = x1 * g1;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (_Float16)p0[e], out[e + 4] = (_Float16)p1[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t k = k0 + e;
                out[e] = (_Float16)(k < q.d_in ? xr[k] * q.g[k] : 0.0f);
            }
        }
        *reinterpret_cast<h8 *>(q.xg + m * q.kpad1 + k0) = out;
    }
}

hipError_t launch_blr_forward(const BlrPlan &pl, const uint32_t *bits_u, const uint32_t *bits_v,
                              const float *h, const float *l, const float *g, const float *x, float *y,
                              void *workspace, bool accumulate, hipStream_t s) {
    char *ws = static_cast<char *>(workspace);
    uint32_t *codes_v = reinterpret_cast<uint32_t *>(ws + pl.off_codes_v);
    uint32_t *codes_u = reinterpret_cast<uint32_t *>(ws + pl.off_codes_u);
    _Float16 *al = reinterpret_cast<_Float16 *>(ws + pl.off_al);
    _Float16 *xg = reinterpret_cast<_Float16 *>(ws + pl.off_xg);
    {
        BlrPrep q{};
        q.bits_v = bits_v, q.bits_u = bits_u, q.codes_v = codes_v, q.codes_u = codes_u;
        q.x = x, q.g = g, q.xg = xg;
        q.words = pl.r / 32, q.M = pl.M, q.r = pl.r, q.d_in = pl.d_in, q.d_out = pl.d_out;
        q.npad1 = pl.npad1, q.kpad1 = pl.kpad1, q.npad2 = pl.npad2, q.kpad2 = pl.kpad2;
        q.nblk_v = ((pl.npad1 / 4 + 255) / 256) * (pl.kpad1 / 16);
        q.nblk_u = (pl.npad2 / 4) * ((pl.kpad2 / 16 + 255) / 256);
        q.xvec = (pl.d_in % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                 ((reinterpret_cast<uintptr_t>(g) & 15) == 0);
        const int64_t nblk_x = (pl.M * (pl.kpad1 / 8) + 255) / 256;
        blr_prep_kernel<<<dim3((unsigned)(q.nblk_v + q.nblk_u + nblk_x)), dim3(256), 0, s>>>(q);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // GEMM1: al[M][kpad2] = f16(l . (xg . S_V)); rows of S_V past r are code 1, so
    // the padded columns come out as 0 (and their factor is 0)
    GemmArgs p1{};
    p1.Ah = xg, p1.lda = pl.kpad1;
    p1.codes = codes_v, p1.kw = pl.kpad1 / 16, p1.scales = nullptr, p1.kbw = 0;
    p1.Ch = al, p1.ldc = pl.kpad2, p1.rowf = l, p1.nrowf = (int)pl.r;
    p1.M = (int)pl.M, p1.N = (int)pl.kpad2, p1.K = (int)pl.kpad1, p1.Kloop = (int)pl.kpad1;
    hipError_t e;
    if (blr_small_tiles(pl.M, pl.kpad2)) {
        e = (pl.kpad1 / 256) % 4 == 0 ? run_gemm<32, 64, 1, 2, 4, 4, kAHalf, false, kEpiHalfScale>(p1, s)
                                      : run_gemm<32, 64, 1, 2, 4, 2, kAHalf, false, kEpiHalfScale>(p1, s);
    } else {
        e = run_gemm<128, 128, 1, 4, 1, 4, kAHalf, false, kEpiHalfScale>(p1, s);
    }
    if (e != hipSuccess) return e;
    // GEMM2: c = al . S_U^T, written as y (see below)
    GemmArgs p2{};
    p2.Ah = al, p2.lda = pl.kpad2;
    p2.codes = codes_u, p2.kw = pl.kpad2 / 16, p2.scales = nullptr, p2.kbw = 0;
    p2.C = y, p2.ldc = pl.d_out, p2.rowf = h;
    p2.M = (int)pl.M, p2.N = (int)pl.d_out, p2.K = (int)pl.kpad2, p2.Kloop = (int)pl.kpad2;
    // y = h . c (later paths of a layer: y = f32(y + f32(h . c)))
    return accumulate ? run_gemm<64, 128, 1, 4, 2, 2, kAHalf, false, kEpiRowScaleAcc, 2, 1>(p2, s)
                      : run_gemm<64, 128, 1, 4, 2, 2, kAHalf, false, kEpiRowScale, 2, 1>(p2, s);
}

// ------------------------------------------------------------------ binary low-rank backward
//
// "cortiq-engine 0.8.43 -- train_mm.rs", module header: for a path with
// a = (x.g) S_V and c = (a.l) S_U^T,
//   dh = sum_t dy.c      db = (dy.h) S_U      dl = sum_t a.db
//   dx' = (db.l) S_V^T   dg = sum_t x.dx'     dx += g.dx'
// with the GEMM inputs staged in f16 under a power-of-two gradient scale gs
// that the GEMM's output factor 1/gs removes again.  a and c are recomputed with
// the forward's kernels and tiles (so with the forward's values); the first
// product also keeps a in f32 for dl.
// The two new products read the bitmaps in the other orientation: S_U^T (rows
// r, contraction d_out) is laid out as S_V is for the forward, and S_V (rows d_in,
// contraction r) as S_U is.  Column sums over the tokens go in two passes, chunks
// of kColChunk tokens then the chunks in order, so results do not depend on timing;
// small chunks give enough threads (columns x chunks) to keep the loads in flight.

constexpr int kColChunk = 16;

BlrBwdPlan blr_bwd_plan(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    BlrBwdPlan p{};
    p.fwd = blr_plan(M, d_in, d_out, r);
    p.kpado = round_up(d_out, kBlrKPad);
    p.npadi = round_up(d_in, kRowPad);
    p.chunks = (M + kColChunk - 1) / kColChunk;
    const int64_t widest = d_in > d_out ? (d_in > r ? d_in : r) : (d_out > r ? d_out : r);
    size_t off = p.fwd.total;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (size_t)round_up((int64_t)(off + bytes), 256);
        return at;
    };
    p.off_codes_ut = take((size_t)p.fwd.npad1 * (p.kpado / 16) * 4);
    p.off_codes_vt = take((size_t)p.npadi * (p.fwd.kpad2 / 16) * 4);
    p.off_a = take((size_t)M * r * 4);
    p.off_c = take((size_t)M * d_out * 4);
    p.off_dyh = take((size_t)M * p.kpado * 2);
    p.off_db = take((size_t)M * r * 4);
    p.off_dbl = take((size_t)M * p.fwd.kpad2 * 2);
    p.off_dxp = take((size_t)M * d_in * 4);
    p.off_part = take((size_t)(p.chunks > 0 ? p.chunks : 1) * widest * 4);
    p.total = off;
    return p;
}

namespace {

enum ColMode { kColStageH = 0, kColDx = 1, kColDxAcc = 2 };

// Pass 1 of a column sum: part[ch][n] = sum over tokens t of chunk ch of
// A[t][n] * B[t][n] (f32, ascending t), for n < N.  Fused with the elementwise
// op that reads the same operand A:
//   kColStageH: H[t][n] = f16(A[t][n] * f[n] * gs) for n < N, 0 for N <= n < ldh;
//   kColDx:     D[t][n] = f[n] * B[t][n];
//   kColDxAcc:  D[t][n] = f32(D[t][n] + f32(f[n] * B[t][n])).
struct ColArgs {
    const float *A, *B, *f;
    float *part;
    _Float16 *H;
    float *D;
    int64_t M, N, lda, ldh;
    float gs;
};

template <int MODE>
__global__ __launch_bounds__(256) void blr_colsum_kernel(ColArgs q) {
#pragma clang fp contract(off)
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t ch = blockIdx.y;
    const int64_t t0 = ch * kColChunk, t1 = t0 + kColChunk < q.M ? t0 + kColChunk : q.M;
    const int64_t ncols = MODE == kColStageH ? q.ldh : q.N;
    if (n >= ncols) return;
    if (n >= q.N) {  // padding columns of the staged operand
        for (int64_t t = t0; t < t1; ++t) q.H[t * q.ldh + n] = (_Float16)0.0f;
        return;
    }
    const float *__restrict__ A = q.A;
    const float *__restrict__ B = q.B;
    _Float16 *__restrict__ H = q.H;
    float *__restrict__ D = q.D;
    const float f = q.f[n];
    float sum = 0.0f;
#pragma unroll 4
    for (int64_t t = t0; t < t1; ++t) {
        const float a = A[t * q.lda + n], b = B[t * q.lda + n];
        sum = sum + a * b;  // product rounded before the sum (no contraction in this kernel)
        if constexpr (MODE == kColStageH) H[t * q.ldh + n] = (_Float16)(a * f * q.gs);
        if constexpr (MODE == kColDx) D[t * q.lda + n] = f * b;
        if constexpr (MODE == kColDxAcc) {
            const float prod = f * b;
            D[t * q.lda + n] = D[t * q.lda + n] + prod;
        }
    }
    q.part[ch * q.N + n] = sum;
}

// Pass 2: out[n] = f32(out[n] + f32(sum over chunks in order of part[ch][n])).
__global__ __launch_bounds__(256) void blr_colsum_finish_kernel(const float *__restrict__ part, float *__restrict__ out,
                                                                int64_t N, int64_t chunks) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    // the loads of a group of chunks are independent: issue them together, then add in order
    float s = 0.0f;
    int64_t ch = 0;
    for (; ch + 16 <= chunks; ch += 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = part[(ch + i) * N + n];
#pragma unroll
        for (int i = 0; i < 16; ++i) s += v[i];
    }
    for (; ch < chunks; ++ch) s += part[ch * N + n];
    out[n] = out[n] + s;
}

template <int MODE>
hipError_t colsum(const ColArgs &q, float *out, int64_t chunks, hipStream_t s) {
    const int64_t ncols = MODE == kColStageH ? q.ldh : q.N;
    blr_colsum_kernel<MODE><<<dim3((unsigned)((ncols + 255) / 256), (unsigned)chunks), dim3(256), 0, s>>>(q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    blr_colsum_finish_kernel<<<dim3((unsigned)((q.N + 255) / 256)), dim3(256), 0, s>>>(q.part, out, q.N, chunks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_blr_backward(const BlrBwdPlan &pb, const uint32_t *bits_u, const uint32_t *bits_v, const float *h,
                               const float *l, const float *g, const float *x, const float *dy, float *dx, float *dh,
                               float *dl, float *dg, float gs, void *workspace, bool accumulate_dx, hipStream_t s) {
    const BlrPlan &pl = pb.fwd;
    const int64_t M = pl.M, d_in = pl.d_in, d_out = pl.d_out, r = pl.r;
    char *ws = static_cast<char *>(workspace);
    auto at = [&](size_t off) { return ws + off; };
    uint32_t *codes_v = reinterpret_cast<uint32_t *>(at(pl.off_codes_v));
    uint32_t *codes_u = reinterpret_cast<uint32_t *>(at(pl.off_codes_u));
    uint32_t *codes_ut = reinterpret_cast<uint32_t *>(at(pb.off_codes_ut));
    uint32_t *codes_vt = reinterpret_cast<uint32_t *>(at(pb.off_codes_vt));
    _Float16 *xg = reinterpret_cast<_Float16 *>(at(pl.off_xg));
    _Float16 *al = reinterpret_cast<_Float16 *>(at(pl.off_al));
    float *a = reinterpret_cast<float *>(at(pb.off_a));
    float *c = reinterpret_cast<float *>(at(pb.off_c));
    _Float16 *dyh = reinterpret_cast<_Float16 *>(at(pb.off_dyh));
    float *db = reinterpret_cast<float *>(at(pb.off_db));
    _Float16 *dbl = reinterpret_cast<_Float16 *>(at(pb.off_dbl));
    float *dxp = reinterpret_cast<float *>(at(pb.off_dxp));
    float *part = reinterpret_cast<float *>(at(pb.off_part));
    hipError_t e;
    // bitmaps in both orientations, and f16(x.g)
    {
        BlrPrep q{};
        q.bits_v = bits_v, q.bits_u = bits_u, q.codes_v = codes_v, q.codes_u = codes_u;
        q.x = x, q.g = g, q.xg = xg;
        q.words = r / 32, q.M = M, q.r = r, q.d_in = d_in, q.d_out = d_out;
        q.npad1 = pl.npad1, q.kpad1 = pl.kpad1, q.npad2 = pl.npad2, q.kpad2 = pl.kpad2;
        q.nblk_v = ((pl.npad1 / 4 + 255) / 256) * (pl.kpad1 / 16);
        q.nblk_u = (pl.npad2 / 4) * ((pl.kpad2 / 16 + 255) / 256);
        q.xvec = (d_in % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                 ((reinterpret_cast<uintptr_t>(g) & 15) == 0);
        const int64_t nblk_x = (M * (pl.kpad1 / 8) + 255) / 256;
        blr_prep_kernel<<<dim3((unsigned)(q.nblk_v + q.nblk_u + nblk_x)), dim3(256), 0, s>>>(q);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        // S_U^T: rows r, contraction d_out (bits along the rows, as S_V's);
        // S_V: rows d_in, contraction r (bits along the contraction, as S_U's)
        BlrPrep t{};
        t.bits_v = bits_u, t.codes_v = codes_ut, t.d_in = d_out, t.kpad1 = pb.kpado, t.npad1 = pl.npad1;
        t.bits_u = bits_v, t.codes_u = codes_vt, t.d_out = d_in, t.kpad2 = pl.kpad2, t.npad2 = pb.npadi;
        t.words = r / 32, t.M = 0, t.r = r;
        t.nblk_v = ((pl.npad1 / 4 + 255) / 256) * (pb.kpado / 16);
        t.nblk_u = (pb.npadi / 4) * ((pl.kpad2 / 16 + 255) / 256);
        blr_prep_kernel<<<dim3((unsigned)(t.nblk_v + t.nblk_u)), dim3(256), 0, s>>>(t);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const bool small = blr_small_tiles(M, pl.kpad2);
    // a = xg . S_V [M][r] in f32, and al = f16(l.a) [M][kpad2] as the forward's GEMM1 writes it
    {
        GemmArgs p{};
        p.Ah = xg, p.lda = pl.kpad1, p.codes = codes_v, p.kw = pl.kpad1 / 16;
        p.C = a, p.ldc = r, p.Ch = al, p.ldch = pl.kpad2, p.rowf = l, p.nrowf = (int)r;
        p.M = (int)M, p.N = (int)pl.kpad2, p.K = (int)pl.kpad1, p.Kloop = (int)pl.kpad1;
        if (small)
            e = (pl.kpad1 / 256) % 4 == 0 ? run_gemm<32, 64, 1, 2, 4, 4, kAHalf, false, kEpiStoreHalf>(p, s)
                                          : run_gemm<32, 64, 1, 2, 4, 2, kAHalf, false, kEpiStoreHalf>(p, s);
        else
            e = run_gemm<128, 128, 1, 4, 1, 4, kAHalf, false, kEpiStoreHalf>(p, s);
        if (e != hipSuccess) return e;
    }
    // c = al . S_U^T   [M][d_out]
    {
        GemmArgs p{};
        p.Ah = al, p.lda = pl.kpad2, p.codes = codes_u, p.kw = pl.kpad2 / 16;
        p.C = c, p.ldc = d_out, p.M = (int)M, p.N = (int)d_out, p.K = (int)pl.kpad2, p.Kloop = (int)pl.kpad2;
        e = run_gemm<64, 128, 1, 4, 2, 2, kAHalf, false, kEpiStore, 2, 1>(p, s);
        if (e != hipSuccess) return e;
    }
    // dh += sum_t dy.c, with dyh = f16(dy.h.gs) staged from the same reads
    {
        ColArgs q{};
        q.A = dy, q.B = c, q.f = h, q.part = part, q.H = dyh, q.M = M, q.N = d_out, q.lda = d_out, q.ldh = pb.kpado;
        q.gs = gs;
        e = colsum<kColStageH>(q, dh, pb.chunks, s);
        if (e != hipSuccess) return e;
    }
    // db = dyh . S_U / gs   [M][r]
    {
        GemmArgs p{};
        p.Ah = dyh, p.lda = pb.kpado, p.codes = codes_ut, p.kw = pb.kpado / 16;
        p.C = db, p.ldc = r, p.M = (int)M, p.N = (int)r, p.K = (int)pb.kpado, p.Kloop = (int)pb.kpado;
        p.alpha = 1.0f / gs;
        if (small)
            e = (pb.kpado / 256) % 4 == 0 ? run_gemm<32, 64, 1, 2, 4, 4, kAHalf, false, kEpiScale>(p, s)
                                          : run_gemm<32, 64, 1, 2, 4, 2, kAHalf, false, kEpiScale>(p, s);
        else
            e = run_gemm<128, 128, 1, 4, 1, 4, kAHalf, false, kEpiScale>(p, s);
        if (e != hipSuccess) return e;
    }
    // dl += sum_t a.db, with dbl = f16(db.l.gs) staged from the same reads
    {
        ColArgs q{};
        q.A = db, q.B = a, q.f = l, q.part = part, q.H = dbl, q.M = M, q.N = r, q.lda = r, q.ldh = pl.kpad2;
        q.gs = gs;
        e = colsum<kColStageH>(q, dl, pb.chunks, s);
        if (e != hipSuccess) return e;
    }
    // dx' = dbl . S_V^T / gs   [M][d_in]
    {
        GemmArgs p{};
        p.Ah = dbl, p.lda = pl.kpad2, p.codes = codes_vt, p.kw = pl.kpad2 / 16;
        p.C = dxp, p.ldc = d_in, p.M = (int)M, p.N = (int)d_in, p.K = (int)pl.kpad2, p.Kloop = (int)pl.kpad2;
        p.alpha = 1.0f / gs;
        e = run_gemm<64, 128, 1, 4, 2, 2, kAHalf, false, kEpiScale, 2, 1>(p, s);
        if (e != hipSuccess) return e;
    }
    // dg += sum_t x.dx', and dx = g.dx' (later paths: dx = f32(dx + f32(g.dx')))
    {
        ColArgs q{};
        q.A = x, q.B = dxp, q.f = g, q.part = part, q.D = dx, q.M = M, q.N = d_in, q.lda = d_in;
        e = accumulate_dx ? colsum<kColDxAcc>(q, dg, pb.chunks, s) : colsum<kColDx>(q, dg, pb.chunks, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tq2
