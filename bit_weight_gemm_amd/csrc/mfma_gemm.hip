// Block-tiled MFMA product C[M][N] = f16(A[M][K] * col[K]) x B[N][K]^T on gfx950,
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
// Tiling: a workgroup of WM x WN waves computes a BM x BN tile, stepping K by 64.
// Each step the workgroup loads the f32 A tile, multiplies by the column factor,
// rounds to f16 and stores it to a double-buffered, XOR-swizzled LDS tile; each
// wave then reads its A fragments from LDS (one 16-byte read per 32-row block
// and 16-wide k slice), loads its B code words straight from memory (one 16-byte
// load per row and step), decodes them, and issues v_mfma_f32_32x32x16_f16.
// The next step's global loads are issued before the current step's MFMAs.
#include <hip/hip_runtime.h>

#include "decode.h"
#include "internal.h"

namespace tq2 {

constexpr int BK = 64;

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

enum Epi { kEpiStore = 0, kEpiRowScale = 1 };

struct GemmArgs {
    const float *A;          // [M][lda] f32
    int64_t lda;
    const float *colf;       // [K] per-k factor or nullptr
    const uint32_t *codes;   // [Npad][kw] code words of B
    int64_t kw;
    const uint16_t *scales;  // [Npad][kbw] f16 scales of B, or nullptr
    int64_t kbw;
    float *C;                // [M][ldc]
    int64_t ldc;
    const float *rowf;       // [N] output factor (kEpiRowScale)
    int M, N, K;             // true sizes; K bounds the A loads
    int Kloop;               // K rounded up to a multiple of 64 (codes are padded)
    int tiles_n;             // number of BN tiles along N
    int a_vec;               // A rows allow 16-byte loads (lda % 4 == 0 and A 16-byte aligned)
};

// 16-byte chunk `kc` (8 halves) of tile row `row`, XOR-swizzled across the row.
__device__ __forceinline__ int lds_off(int row, int kc) { return row * BK + ((kc ^ (row & 7)) << 3); }

template <int BM, int BN, int WM, int WN, bool KGUARD, bool COLF, bool SCALED, int EPI>
__global__ __launch_bounds__(WM *WN * 64) void mfma_gemm_kernel(GemmArgs p) {
    constexpr int T = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MB = WTM / 32, NB = WTN / 32;
    constexpr int CHUNKS = BM * (BK / 8);
    constexpr int CPT = CHUNKS / T;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(CHUNKS % T == 0, "A tile must split evenly over the threads");

    __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * BK];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int lrow = lane & 31, hk = lane >> 5;

    // Tile order: consecutive workgroups walk N first, so the ones sharing an A
    // row-block run together and reuse it from L2.
    const int tile = blockIdx.x;
    const int m0 = (tile / p.tiles_n) * BM;
    const int n0 = (tile % p.tiles_n) * BN;

    f16x acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f16x{};

    // ---- prefetch registers
    float areg[CPT][8];
    u4 breg[NB];
    _Float16 dreg[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) dreg[nb] = (_Float16)1.0f;

    auto load_a = [&](int k0) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int chunk = tid + c * T;
            const int row = chunk >> 3, kc = chunk & 7;
            const int gm = m0 + row, gk = k0 + kc * 8;
            if (gm < p.M && (!KGUARD || (p.a_vec && gk + 8 <= p.K))) {
                const f4 *src = reinterpret_cast<const f4 *>(p.A + (int64_t)gm * p.lda + gk);
                const f4 v0 = src[0], v1 = src[1];
                areg[c][0] = v0.x, areg[c][1] = v0.y, areg[c][2] = v0.z, areg[c][3] = v0.w;
                areg[c][4] = v1.x, areg[c][5] = v1.y, areg[c][6] = v1.z, areg[c][7] = v1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    areg[c][e] = (gm < p.M && KGUARD && gk + e < p.K) ? p.A[(int64_t)gm * p.lda + gk + e] : 0.0f;
            }
        }
    };
    auto load_b = [&](int k0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int64_t n = n0 + wn * WTN + nb * 32 + lrow;
            breg[nb] = *reinterpret_cast<const u4 *>(p.codes + n * p.kw + (k0 >> 4));
            if constexpr (SCALED) dreg[nb] = __builtin_bit_cast(_Float16, p.scales[n * p.kbw + k0 / kBlock]);
        }
    };
    auto store_a = [&](int buf, int k0) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int chunk = tid + c * T;
            const int row = chunk >> 3, kc = chunk & 7;
            h8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = areg[c][e];
                if constexpr (COLF) {
                    const int gk = k0 + kc * 8 + e;
                    a = (!KGUARD || gk < p.K) ? a * p.colf[gk] : 0.0f;
                }
                v[e] = (_Float16)a;
            }
            *reinterpret_cast<h8 *>(&As[buf][lds_off(row, kc)]) = v;
        }
    };

    load_a(0);
    load_b(0);
    int buf = 0;
    for (int k0 = 0; k0 < p.Kloop; k0 += BK, buf ^= 1) {
        store_a(buf, k0);
        u4 bcur[NB];
        _Float16 dcur[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bcur[nb] = breg[nb], dcur[nb] = dreg[nb];
        __syncthreads();
        if (k0 + BK < p.Kloop) {
            load_a(k0 + BK);
            load_b(k0 + BK);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h8 a[MB], b[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = wm * WTM + mb * 32 + lrow;
                a[mb] = *reinterpret_cast<const h8 *>(&As[buf][lds_off(row, 2 * j + hk)]);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                b[nb] = half_group_m1(bcur[nb][j], hk);
                if constexpr (SCALED) b[nb] = b[nb] * dcur[nb];
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mb], b[nb], acc[mb][nb], 0, 0, 0);
        }
    }

    // ---- epilogue: lane holds column lrow, rows 8*(r/4) + 4*hk + r%4 of each block
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int gn = n0 + wn * WTN + nb * 32 + lrow;
            if (gn >= p.N) continue;
            const float rf = (EPI == kEpiRowScale) ? p.rowf[gn] : 1.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm * WTM + mb * 32 + 8 * (r >> 2) + 4 * hk + (r & 3);
                if (gm < p.M) {
                    const float v = acc[mb][nb][r];
                    p.C[(int64_t)gm * p.ldc + gn] = (EPI == kEpiRowScale) ? rf * v : v;
                }
            }
        }
}

template <int BM, int BN, int WM, int WN, bool KGUARD, bool COLF, bool SCALED, int EPI>
static hipError_t run_gemm(GemmArgs p, int64_t npad, hipStream_t s) {
    p.tiles_n = (int)((p.N + BN - 1) / BN);  // tiles_n * BN <= npad, so B rows stay in bounds
    (void)npad;
    const int64_t tiles_m = (p.M + BM - 1) / BM;
    const int64_t tiles = tiles_m * p.tiles_n;
    mfma_gemm_kernel<BM, BN, WM, WN, KGUARD, COLF, SCALED, EPI>
        <<<dim3((unsigned)tiles), dim3(WM * WN * 64), 0, s>>>(p);
    return hipGetLastError();
}

// ------------------------------------------------------------------ ternary GEMM, large M

hipError_t launch_gemm_mfma(const DevWeight &w, const float *x, float *y, int64_t M, hipStream_t s) {
    GemmArgs p{};
    p.A = x;
    p.lda = w.K;
    p.colf = nullptr;
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
    p.a_vec = 1;
    if (M <= 64) return run_gemm<32, 256, 1, 4, false, false, true, kEpiStore>(p, w.Npad, s);
    return run_gemm<128, 256, 1, 4, false, false, true, kEpiStore>(p, w.Npad, s);
}

// ------------------------------------------------------------------ binary low-rank forward

static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

constexpr int kBlrBN = 64;

BlrPlan blr_plan(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    BlrPlan p{};
    p.M = M, p.d_in = d_in, p.d_out = d_out, p.r = r;
    p.kpad1 = round_up(d_in, BK);
    p.kpad2 = round_up(r, BK);
    p.npad1 = round_up(r, kRowPad);
    p.npad2 = round_up(d_out, kRowPad);
    size_t off = 0;
    p.off_codes_v = off;
    off += (size_t)p.npad1 * (p.kpad1 / 16) * 4;
    off = (size_t)round_up((int64_t)off, 256);
    p.off_codes_u = off;
    off += (size_t)p.npad2 * (p.kpad2 / 16) * 4;
    off = (size_t)round_up((int64_t)off, 256);
    p.off_a = off;
    off += (size_t)M * r * 4;
    p.total = (size_t)round_up((int64_t)off, 256);
    return p;
}

// Sign bitmaps -> code words (set bit -> code 2 = +1, clear -> code 0 = -1,
// padding -> code 1 = 0) in the device layout, with row index `n` and
// contraction index `k`:
//   TRANS = false: sign(n, k) = bit k of bits[n][k/32]   (S_U: n = output i, k = rank)
//   TRANS = true:  sign(n, k) = bit n of bits[k][n/32]   (S_V: n = rank, k = input j)
template <bool TRANS>
__global__ __launch_bounds__(256) void bits_to_codes_kernel(const uint32_t *__restrict__ bits, int64_t words,
                                                            uint32_t *__restrict__ codes, int64_t n_real,
                                                            int64_t k_real, int64_t n_pad, int64_t k_pad) {
    const int64_t kw = k_pad / 16;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_pad * kw) return;
    const int64_t n = gid / kw, g = gid % kw;
    uint32_t out = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int64_t k = g * 16 + e;
        uint32_t code = 1;
        if (n < n_real && k < k_real) {
            const uint32_t b = TRANS ? (bits[k * words + (n >> 5)] >> (n & 31)) & 1u
                                     : (bits[n * words + (k >> 5)] >> (k & 31)) & 1u;
            code = b ? 2u : 0u;
        }
        out |= code << (2 * (e >> 1) + 16 * (e & 1));
    }
    codes[n * kw + g] = out;
}

hipError_t launch_blr_forward(const BlrPlan &pl, const uint32_t *bits_u, const uint32_t *bits_v,
                              const float *h, const float *l, const float *g, const float *x, float *y,
                              void *workspace, hipStream_t s) {
    char *ws = static_cast<char *>(workspace);
    uint32_t *codes_v = reinterpret_cast<uint32_t *>(ws + pl.off_codes_v);
    uint32_t *codes_u = reinterpret_cast<uint32_t *>(ws + pl.off_codes_u);
    float *a = reinterpret_cast<float *>(ws + pl.off_a);
    const int64_t words = pl.r / 32;

    {
        const int64_t tot = pl.npad1 * (pl.kpad1 / 16);
        bits_to_codes_kernel<true><<<dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s>>>(
            bits_v, words, codes_v, pl.r, pl.d_in, pl.npad1, pl.kpad1);
        const int64_t tot2 = pl.npad2 * (pl.kpad2 / 16);
        bits_to_codes_kernel<false><<<dim3((unsigned)((tot2 + 255) / 256)), dim3(256), 0, s>>>(
            bits_u, words, codes_u, pl.d_out, pl.r, pl.npad2, pl.kpad2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // GEMM1: a[M][r] = f16(x.g) . S_V
    GemmArgs p1{};
    p1.A = x, p1.lda = pl.d_in, p1.colf = g;
    p1.codes = codes_v, p1.kw = pl.kpad1 / 16, p1.scales = nullptr, p1.kbw = 0;
    p1.C = a, p1.ldc = pl.r, p1.rowf = nullptr;
    p1.M = (int)pl.M, p1.N = (int)pl.r, p1.K = (int)pl.d_in, p1.Kloop = (int)pl.kpad1;
    p1.a_vec = (pl.d_in % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    hipError_t e = run_gemm<64, kBlrBN, 2, 2, true, true, false, kEpiStore>(p1, pl.npad1, s);
    if (e != hipSuccess) return e;
    // GEMM2: y[M][d_out] = h . (f16(a.l) . S_U^T)
    GemmArgs p2{};
    p2.A = a, p2.lda = pl.r, p2.colf = l;
    p2.codes = codes_u, p2.kw = pl.kpad2 / 16, p2.scales = nullptr, p2.kbw = 0;
    p2.C = y, p2.ldc = pl.d_out, p2.rowf = h;
    p2.M = (int)pl.M, p2.N = (int)pl.d_out, p2.K = (int)pl.r, p2.Kloop = (int)pl.kpad2;
    p2.a_vec = 1;
    return run_gemm<64, kBlrBN, 2, 2, true, true, false, kEpiRowScale>(p2, pl.npad2, s);
}

}  // namespace tq2
