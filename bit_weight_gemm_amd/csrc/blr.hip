// Binary low-rank layer ("cortiq-engine 0.8.43 -- train_mm.rs", module header,
// blr_forward / blr_backward): the layer's products on the block-tiled MFMA
// kernel of mfma_gemm.h, which reads the sign bitmaps as the caller holds them.
#include "mfma_gemm.h"

namespace tq2 {

// ------------------------------------------------------------------ binary low-rank forward

static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Two products, each one launch of the MFMA kernel, expanding the sign bitmaps
// inside the GEMM as the page's mm_bits does:
//   GEMM1 (M x r, K = d_in): A = f16(x.g) staged from f32 x and g in the
//     kernel, B = S_V from bits_v, whose bits run along r (kBSignT: the tile is
//     transposed in the LDS staging); its epilogue writes f16(l.a), 0 past r, in
//     the perm32 k order that GEMM2's decode reads.
//   GEMM2 (M x d_out, K = r): A = that f16 operand, B = S_U from bits_u, whose
//     bits run along r (kBSign); its epilogue writes y = h.c.
// Small M takes 32 x 64 tiles of GEMM1 (eight waves, four k groups) so that
// enough workgroups stream the long K without splitting it; larger M takes
// 128 x 128 tiles.
constexpr int kBlrKPad = 512;          // GEMM1's K padding: whole pipeline rounds of either tile
constexpr int kBlr2Step = 2 * 2 * BK;  // GEMM2: 128-wide steps, two stages

static bool blr_small_tiles(int64_t M, int64_t kpad2) { return ((M + 31) / 32) * (kpad2 / 64) < 2048; }

// GEMM1 with its contraction (d_in) split over workgroups: 32 x 128 tiles of
// 256-wide steps, two steps per pipeline round, so each chunk of d_in is a
// multiple of 512.  With the small tiles a workgroup stages its 32 rows of x
// (f32, multiplied by g and rounded to f16) over all of d_in; split two (or
// four) ways over tiles twice as wide, it stages half (a quarter) of them for
// the same MFMA work, and a last launch adds the chunks' partial products in
// order (blr_g1_finish_kernel), which costs ~3 us per layer.  Measured per layer
// call (unsplit / split, us) at d_in = 4096, r = 1024: M=128 22.4 / 19.3, M=256
// 23.5 / 22.7, M=512 25.9 / 26.3, M=1024 44.9 / 42.6; at d_in = 2048, r = 512:
// M=512 15.6 / 17.0, M=300 15.0 / 15.1.  So the split is used with d_in >= 4096
// where the 32 x 64 tiles would not make exactly one full round of workgroups
// (fewer than 192, or more than 256), and the split grid fills between half and
// two times the CUs.
constexpr int kG1SplitRound = 512;
static int64_t gemm1_ksplit(int64_t M, int64_t kpad1, int64_t kpad2) {
    if (!blr_small_tiles(M, kpad2) || kpad2 % 128 != 0 || kpad1 < 4096) return 1;
    const int64_t unsplit = ((M + 31) / 32) * (kpad2 / 64);
    if (unsplit >= 192 && unsplit <= 256) return 1;
    const int64_t tiles = ((M + 31) / 32) * (kpad2 / 128);
    for (int64_t ks = 2; ks <= 4; ks *= 2)
        if (kpad1 % (ks * kG1SplitRound) == 0 && tiles * ks >= 128 && tiles * ks <= 512) return ks;
    return 1;
}

// An f16 A operand within 2 GB (rows of the last tile included) is read through
// a buffer resource with 32-bit offsets.
static bool half_buf(const GemmArgs &p) { return ((int64_t)p.M + 256) * p.lda * 2 < ((int64_t)1 << 31); }

// Products with the long contraction (GEMM1 over d_in, and the backward's db over
// d_out), of M x r outputs, B a bitmap whose bits run along the outputs:
// 32 x 64 tiles when they are few, else 128 x 128 tiles.  256-wide steps with two
// A register stages, for A staged from f32 x (x.g rounded in the kernel: GEMM1 at
// M=512, d_in=4096, r=1024 16.2 against 19.1 us alone with 512-wide steps and one
// stage) and for an f16 A alike (db at the same shape: 12.9 against 13.9 us).
template <int EPI, int AMODE>
static hipError_t gemm_long_k(const GemmArgs &p, bool small, hipStream_t s) {
    constexpr bool half_a = AMODE == kAHalf || AMODE == kAHalfBuf;
    // (f32 pieces of x take twice the registers of f16 ones: two A register stages)
    if (!small) return run_gemm<128, 128, 1, 4, 1, 4, AMODE, false, EPI, 4, half_a ? 4 : 2, 1, kBSignT>(p, s);
    return run_gemm<32, 64, 1, 2, 4, 2, AMODE, false, EPI, 2, 2, 1, kBSignT>(p, s);
}
// Products with the short contraction r (GEMM2, and the backward's c and dx'), B
// a bitmap whose bits run along r: 64 x 128 tiles of eight waves (two row waves
// by four column waves, one k group taking two 64-wide slices of each 128-wide
// step), A loaded two steps ahead.  With only eight steps per tile, two k groups
// (one slice each) cost more in their closing sums than their shorter loop saves
// (GEMM2 at M=512, d_out=4096, r=1024: 10.6 against 10.85 us alone).
template <int EPI>
static hipError_t gemm_short_k(const GemmArgs &p, hipStream_t s) {
    if (half_buf(p)) return run_gemm<64, 128, 2, 4, 1, 2, kAHalfBuf, false, EPI, 2, 2, 2, kBSign>(p, s);
    return run_gemm<64, 128, 2, 4, 1, 2, kAHalf, false, EPI, 2, 2, 2, kBSign>(p, s);
}

BlrPlan blr_plan(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    BlrPlan p{};
    p.M = M, p.d_in = d_in, p.d_out = d_out, p.r = r;
    p.kpad1 = round_up(d_in, kBlrKPad);
    p.kpad2 = round_up(r, kBlr2Step);
    p.ksplit1 = gemm1_ksplit(M, p.kpad1, p.kpad2);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (size_t)round_up((int64_t)(off + bytes), 256);
        return at;
    };
    p.off_al = take((size_t)M * p.kpad2 * 2);
    p.off_part1 = p.ksplit1 > 1 ? take((size_t)p.ksplit1 * M * p.kpad2 * 4) : 0;
    p.total = off;
    return p;
}

// GEMM1's arguments: A = f16(x.g) from f32 x, B = S_V (bits_v: d_in rows of r/32
// words), N = the padded rank (columns past r come out as 0 through their factor).
static GemmArgs gemm1_args(const BlrPlan &pl, const uint32_t *bits_v, const float *g, const float *x) {
    GemmArgs p{};
    p.A = x, p.lda = pl.d_in, p.g = g;
    p.bits = bits_v, p.ldb = pl.r / 32, p.nbits = (int)(pl.r / 32), p.kbits = (int)pl.d_in;
    p.M = (int)pl.M, p.N = (int)pl.kpad2, p.K = (int)pl.d_in, p.Kloop = (int)pl.kpad1;
    return p;
}

// x through a buffer resource with no K tail: d_in a multiple of every step of
// GEMM1's tiles, 16-byte aligned rows and g, x within 2 GB.
static bool xg_vector(const BlrPlan &pl, const float *x, const float *g) {
    return pl.d_in % kBlrKPad == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(g) & 15) == 0 && (pl.M + 256) * pl.d_in * 4 < ((int64_t)1 << 31);
}

template <int EPI>
static hipError_t run_gemm1(const GemmArgs &p, const BlrPlan &pl, bool vec, hipStream_t s) {
    const bool small = blr_small_tiles(pl.M, pl.kpad2);
    return vec ? gemm_long_k<EPI, kAXG>(p, small, s) : gemm_long_k<EPI, kAXGS>(p, small, s);
}

namespace {

// The epilogue of GEMM1 when its contraction is split: per row m and 16-byte
// unit of al's row (columns n0..n0+3 and n0+16..n0+19 of a group of 32, which
// perm32 puts next to each other), the chunks' partial products added in chunk
// order, then al[m][perm32(n)] = f16(f*a) with f = l[n] (0 past r), as the
// unsplit product's kEpiHalfScaleP writes it, and a[m][n] itself (n < r) when kept.
struct G1FinishArgs {
    const float *part;  // [KS][M][kpad2]
    int64_t cks;        // elements between chunks (M*kpad2)
    int64_t M, kpad2, r;
    const float *l;     // [r]
    _Float16 *al;       // [M][kpad2]
    float *a;           // [M][r], or nullptr
};

template <int KS>
__global__ __launch_bounds__(256) void blr_g1_finish_kernel(G1FinishArgs q) {
#pragma clang fp contract(off)
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t units = q.kpad2 / 8;
    const int64_t m = tid / units, u = tid % units;
    if (m >= q.M) return;
    const int64_t n0 = (u >> 2) * 32 + 4 * (u & 3);
    const float *pp = q.part + m * q.kpad2 + n0;
    f4 lo[KS], hi[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        lo[j] = *reinterpret_cast<const f4 *>(pp + j * q.cks);
        hi[j] = *reinterpret_cast<const f4 *>(pp + j * q.cks + 16);
    }
    // r % 32 == 0: the group of 32 columns is all below r or all padding
    const bool real = n0 < q.r;
    const int64_t nl = real ? n0 : 0;
    f4 f0, f1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f0[i] = q.l[nl + i];
        f1[i] = q.l[nl + 16 + i];
    }
    f4 s0 = lo[0], s1 = hi[0];
#pragma unroll
    for (int j = 1; j < KS; ++j) {
        s0 = s0 + lo[j];
        s1 = s1 + hi[j];
    }
    if (!real) f0 = f4{}, f1 = f4{};
    const f4 o0 = f0 * s0, o1 = f1 * s1;
    const h8 out = {(_Float16)o0[0], (_Float16)o1[0], (_Float16)o0[1], (_Float16)o1[1],
                    (_Float16)o0[2], (_Float16)o1[2], (_Float16)o0[3], (_Float16)o1[3]};
    *reinterpret_cast<h8 *>(q.al + m * q.kpad2 + 8 * u) = out;
    if (q.a && real) {
        float *ar = q.a + m * q.r + n0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ar[i] = s0[i];
            ar[16 + i] = s1[i];
        }
    }
}

}  // namespace

// GEMM1 with its epilogue: al = f16(l.a) [M][kpad2] (perm32 order, 0 in the
// columns past r) and, when `a` is given, a [M][r] itself in f32.
static hipError_t gemm1(const BlrPlan &pl, const uint32_t *bits_v, const float *l, const float *g, const float *x,
                        _Float16 *al, float *a, char *ws, hipStream_t s) {
    const bool vec = xg_vector(pl, x, g);
    GemmArgs p = gemm1_args(pl, bits_v, g, x);
    if (pl.ksplit1 > 1) {
        float *part = reinterpret_cast<float *>(ws + pl.off_part1);
        p.C = part, p.ldc = pl.kpad2, p.ksplit = (int)pl.ksplit1, p.cks = pl.M * pl.kpad2;
        const hipError_t e = vec ? run_gemm<32, 128, 1, 4, 2, 2, kAXG, false, kEpiStore, 2, 2, 2, kBSignT>(p, s)
                                 : run_gemm<32, 128, 1, 4, 2, 2, kAXGS, false, kEpiStore, 2, 2, 2, kBSignT>(p, s);
        if (e != hipSuccess) return e;
        G1FinishArgs q{};
        q.part = part, q.cks = pl.M * pl.kpad2, q.M = pl.M, q.kpad2 = pl.kpad2, q.r = pl.r;
        q.l = l, q.al = al, q.a = a;
        const unsigned wgs = (unsigned)((pl.M * (pl.kpad2 / 8) + 255) / 256);
        if (pl.ksplit1 == 4)
            blr_g1_finish_kernel<4><<<dim3(wgs), dim3(256), 0, s>>>(q);
        else
            blr_g1_finish_kernel<2><<<dim3(wgs), dim3(256), 0, s>>>(q);
        return hipGetLastError();
    }
    p.rowf = l, p.nrowf = (int)pl.r;
    if (a) {
        p.C = a, p.ldc = pl.r, p.Ch = al, p.ldch = pl.kpad2;
        return run_gemm1<kEpiStoreHalfP>(p, pl, vec, s);
    }
    p.Ch = al, p.ldc = pl.kpad2;
    return run_gemm1<kEpiHalfScaleP>(p, pl, vec, s);
}

// GEMM2's arguments: A = f16(l.a) [M][kpad2] (perm32 order), B = S_U (bits_u:
// d_out rows of r/32 words).
static GemmArgs gemm2_args(const BlrPlan &pl, const uint32_t *bits_u, const _Float16 *al) {
    GemmArgs p{};
    p.Ah = al, p.lda = pl.kpad2;
    p.bits = bits_u, p.ldb = pl.r / 32, p.nbits = (int)pl.d_out, p.kbits = (int)(pl.r / 32);
    p.M = (int)pl.M, p.N = (int)pl.d_out, p.K = (int)pl.kpad2, p.Kloop = (int)pl.kpad2;
    return p;
}

hipError_t launch_blr_forward(const BlrPlan &pl, const uint32_t *bits_u, const uint32_t *bits_v,
                              const float *h, const float *l, const float *g, const float *x, float *y,
                              void *workspace, bool accumulate, float *save_a, float *save_c, hipStream_t s) {
    char *ws = static_cast<char *>(workspace);
    _Float16 *al = reinterpret_cast<_Float16 *>(ws + pl.off_al);
    const bool save = save_a != nullptr;
    // GEMM1: al[M][kpad2] = f16(l . (f16(x.g) . S_V)), 0 in the columns past r
    // (saving: also a[M][r] in f32, as the backward's recomputation writes it)
    const hipError_t e = gemm1(pl, bits_v, l, g, x, al, save_a, ws, s);
    if (e != hipSuccess) return e;
    // GEMM2: y = h . (al . S_U^T) (later paths of a layer: y = f32(y + f32(h . c)));
    // saving: also c[M][d_out] itself
    GemmArgs p2 = gemm2_args(pl, bits_u, al);
    p2.C = y, p2.ldc = pl.d_out, p2.rowf = h;
    if (save) {
        p2.Cs = save_c, p2.ldcs = pl.d_out;
        return accumulate ? gemm_short_k<kEpiRowScaleAccSave>(p2, s) : gemm_short_k<kEpiRowScaleSave>(p2, s);
    }
    return accumulate ? gemm_short_k<kEpiRowScaleAcc>(p2, s) : gemm_short_k<kEpiRowScale>(p2, s);
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
// The two new products read the bitmaps in the other orientation: db contracts
// over d_out, down the rows of bits_u (kBSignT, as GEMM1 reads bits_v), and dx'
// over r, along the rows of bits_v (kBSign, as GEMM2 reads bits_u).  The column
// sums over the tokens and the f16 staging of each next product's input are
// done in the epilogues of the products that produce their operands (the
// kEpiBwd* modes of mfma_gemm.h): c's epilogue reads dy and keeps the partial
// sums of dy.c per block of 32 tokens and writes f16(dy.h.gs) (perm4 order, for
// db); db's reads a, keeps those of a.db and writes f16(db.l.gs) (perm32 order,
// for dx'); dx''s reads x, keeps those of x.dx' and writes dx.  A last launch
// adds each gradient's partial sums, the blocks in order.  So c, db and dx'
// never go to memory, and the backward is five launches.

static int64_t row_blocks(int64_t M) { return (M + 31) / 32; }

BlrBwdPlan blr_bwd_plan(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    BlrBwdPlan p{};
    p.fwd = blr_plan(M, d_in, d_out, r);
    p.kpado = round_up(d_out, kBlrKPad);
    p.blocks = row_blocks(M);
    size_t off = p.fwd.total;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (size_t)round_up((int64_t)(off + bytes), 256);
        return at;
    };
    p.off_a = take((size_t)M * r * 4);
    p.off_dyh = take((size_t)M * p.kpado * 2);
    p.off_dbl = take((size_t)M * p.fwd.kpad2 * 2);
    const size_t nb = (size_t)(p.blocks > 0 ? p.blocks : 1);
    p.off_part_dh = take(nb * d_out * 4);
    p.off_part_dl = take(nb * r * 4);
    p.off_part_dg = take(nb * d_in * 4);
    p.total = off;
    return p;
}

namespace {

// With the forward's c saved: for each block of 32 tokens and column n < N
// (d_out padded), the partial sum of dy.c over the block's tokens, in the order
// c's epilogue (kEpiBwdC) adds them (tokens 8i+j, then 8i+4+j, for i, j = 0..3,
// each half summed in that order and the halves added), so the same bits; and
// dyh[t][perm4(n)] = f16((dy*h)*gs), 0 for the padding columns n >= d_out.
struct DycArgs {
    const float *dy, *c, *h;   // dy, c [M][d_out]; h [d_out]
    _Float16 *dyh;             // [M][ldh]
    float *part;               // [blocks][d_out]
    int64_t M, d_out, N, ldh, blocks;
    float gs;
};

// Thread (column group, half, block): four consecutive columns (W = 4, 16-byte
// loads of dy and c, one 8-byte store of dyh per token; d_out % 4 == 0) or one
// column (W = 1), and the 16 tokens of one half of a block of 32; the two
// halves of a block are adjacent lanes, whose sums are added through a lane
// exchange (addition commutes, so either lane's sum has the same bits).  Every
// value of dy and c a thread needs is loaded before any is used.
template <int W, bool FULL>
__device__ __forceinline__ void dyc_half(const DycArgs &q, int64_t b, int hk, int64_t n0, bool real) {
#pragma clang fp contract(off)
    typedef float fw __attribute__((ext_vector_type(W)));
    typedef _Float16 hw __attribute__((ext_vector_type(W)));
    // rows of this half: 32b + 8(r/4) + 4hk + r%4; FULL: all 16 below M.  The
    // loads are unconditional (padding columns read column 0 and rows past M
    // read row M-1, then the values are replaced by 0), so they need no branches
    // and go out together.
    const int64_t nc = real ? n0 : 0;
    const int64_t t0 = 32 * b + 4 * hk;
    _Float16 *dyh = q.dyh + t0 * q.ldh + n0;
    fw e[16], v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t dt = 8 * (r >> 2) + (r & 3);
        const bool live = real && (FULL || t0 + dt < q.M);
        const int64_t t = FULL ? t0 + dt : (t0 + dt < q.M ? t0 + dt : q.M - 1);
        const fw ev = *reinterpret_cast<const fw *>(q.dy + t * q.d_out + nc);
        const fw cv = *reinterpret_cast<const fw *>(q.c + t * q.d_out + nc);
        e[r] = live ? ev : fw{};
        v[r] = live ? cv : fw{};
    }
    const fw hf = *reinterpret_cast<const fw *>(q.h + nc);
    const fw f = real ? hf : fw{};
    fw psum{};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t dt = 8 * (r >> 2) + (r & 3);
        if (FULL || t0 + dt < q.M) {
            psum = psum + e[r] * v[r];
            const fw o = (e[r] * f) * q.gs;
            if constexpr (W == 4) {
                const hw out = {(_Float16)o[0], (_Float16)o[2], (_Float16)o[1], (_Float16)o[3]};  // perm4 order
                *reinterpret_cast<hw *>(dyh + dt * q.ldh) = out;
            } else {
                dyh[dt * q.ldh + (perm4((int)n0) - n0)] = (_Float16)o[0];
            }
        }
    }
    fw other;
#pragma unroll
    for (int i = 0; i < W; ++i) other[i] = __shfl_xor(psum[i], 1);
    if (real && hk == 0) *reinterpret_cast<fw *>(q.part + b * q.d_out + n0) = psum + other;
}

template <int W>
__global__ __launch_bounds__(256) void blr_dyc_kernel(DycArgs q) {
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int hk = (int)(tid & 1);
    const int64_t groups = q.N / W;
    const int64_t n0 = ((tid >> 1) % groups) * W;
    const int64_t b = (tid >> 1) / groups;
    const bool real = n0 < q.d_out;  // d_out % W == 0: the group is all real or all padding
    if (b >= q.blocks) return;       // whole lane pairs leave together
    // blocks of 32 tokens below M take the path without per-token checks
    if (32 * b + 32 <= q.M)
        dyc_half<W, true>(q, b, hk, n0, real);
    else
        dyc_half<W, false>(q, b, hk, n0, real);
}

// out[n] = f32(out[n] + f32(sum over row blocks b in order of part[b][n])) for the
// three gradients of a path (dh: d_out columns, dl: r, dg: d_in), one thread per
// column.  Each gradient's columns start a workgroup, so a workgroup's gradient is
// the same for all its threads and its pointers come from scalar loads; out[n] is
// loaded together with the partial sums of a group of blocks, which are then
// added in order.
struct FinishJob {
    const float *part;
    float *out;
    int64_t N;
};
struct FinishArgs {
    FinishJob job[3];
    int64_t blocks;
    unsigned wg1, wg2;  // first workgroups of gradients 1 and 2
};

__global__ __launch_bounds__(256) void blr_finish_kernel(FinishArgs q) {
#pragma clang fp contract(off)
    const unsigned wg = blockIdx.x;
    const int j = wg >= q.wg2 ? 2 : wg >= q.wg1 ? 1 : 0;
    const unsigned first = j == 2 ? q.wg2 : j == 1 ? q.wg1 : 0u;
    const float *__restrict__ part = q.job[j].part;
    float *__restrict__ out = q.job[j].out;
    const int64_t N = q.job[j].N;
    const int64_t n = (int64_t)(wg - first) * 256 + threadIdx.x;
    if (n >= N) return;
    const float o = out[n];
    float s = 0.0f;
    int64_t b = 0;
    for (; b + 16 <= q.blocks; b += 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = part[(b + i) * N + n];
#pragma unroll
        for (int i = 0; i < 16; ++i) s = s + v[i];
    }
    for (; b < q.blocks; ++b) s = s + part[b * N + n];
    out[n] = o + s;
}

}  // namespace

// db, dx' and the finish of a path's backward, from dyh and a (launches 3 to 5).
static hipError_t backward_tail(const BlrBwdPlan &pb, const uint32_t *bits_u, const uint32_t *bits_v, const float *l,
                                const float *g, const float *x, const float *a, float *dx, float *dh, float *dl,
                                float *dg, float gs, char *ws, bool accumulate_dx, bool small, hipStream_t s) {
    const BlrPlan &pl = pb.fwd;
    const int64_t M = pl.M, d_in = pl.d_in, d_out = pl.d_out, r = pl.r;
    _Float16 *dyh = reinterpret_cast<_Float16 *>(ws + pb.off_dyh);
    _Float16 *dbl = reinterpret_cast<_Float16 *>(ws + pb.off_dbl);
    float *part_dh = reinterpret_cast<float *>(ws + pb.off_part_dh);
    float *part_dl = reinterpret_cast<float *>(ws + pb.off_part_dl);
    float *part_dg = reinterpret_cast<float *>(ws + pb.off_part_dg);
    hipError_t e;
    // db = dyh . S_U / gs (not stored; contraction over d_out, down the rows of bits_u):
    // partial sums of a.db, and dbl = f16(db.l.gs) [M][kpad2] (perm32 order)
    {
        GemmArgs p{};
        p.Ah = dyh, p.lda = pb.kpado;
        p.bits = bits_u, p.ldb = r / 32, p.nbits = (int)(r / 32), p.kbits = (int)d_out;
        p.M = (int)M, p.N = (int)pl.kpad2, p.K = (int)pb.kpado, p.Kloop = (int)pb.kpado;
        p.alpha = 1.0f / gs, p.nrowf = (int)r, p.rowf = l;
        p.ea = a, p.ldea = r, p.part = part_dl, p.Ch = dbl, p.ldch = pl.kpad2, p.gs = gs;
        e = half_buf(p) ? gemm_long_k<kEpiBwdDb, kAHalfBuf>(p, small, s) : gemm_long_k<kEpiBwdDb, kAHalf>(p, small, s);
        if (e != hipSuccess) return e;
    }
    // dx' = dbl . S_V^T / gs (not stored; contraction over r, along the rows of bits_v):
    // partial sums of x.dx', and dx = g.dx' (later paths: dx = f32(dx + f32(g.dx')))
    {
        GemmArgs p{};
        p.Ah = dbl, p.lda = pl.kpad2;
        p.bits = bits_v, p.ldb = r / 32, p.nbits = (int)d_in, p.kbits = (int)(r / 32);
        p.C = dx, p.ldc = d_in, p.M = (int)M, p.N = (int)d_in, p.K = (int)pl.kpad2, p.Kloop = (int)pl.kpad2;
        p.alpha = 1.0f / gs, p.nrowf = (int)d_in, p.rowf = g;
        p.ea = x, p.ldea = d_in, p.part = part_dg;
        e = accumulate_dx ? gemm_short_k<kEpiBwdDxAcc>(p, s) : gemm_short_k<kEpiBwdDx>(p, s);
        if (e != hipSuccess) return e;
    }
    // dh, dl, dg += their partial sums, the row blocks in order
    FinishArgs q{};
    q.job[0] = FinishJob{part_dh, dh, d_out};
    q.job[1] = FinishJob{part_dl, dl, r};
    q.job[2] = FinishJob{part_dg, dg, d_in};
    q.blocks = pb.blocks;
    const unsigned w0 = (unsigned)((d_out + 255) / 256), w1 = (unsigned)((r + 255) / 256),
                   w2 = (unsigned)((d_in + 255) / 256);
    q.wg1 = w0, q.wg2 = w0 + w1;
    blr_finish_kernel<<<dim3(w0 + w1 + w2), dim3(256), 0, s>>>(q);
    return hipGetLastError();
}

hipError_t launch_blr_backward(const BlrBwdPlan &pb, const uint32_t *bits_u, const uint32_t *bits_v, const float *h,
                               const float *l, const float *g, const float *x, const float *dy, float *dx, float *dh,
                               float *dl, float *dg, float gs, void *workspace, bool accumulate_dx, hipStream_t s) {
    const BlrPlan &pl = pb.fwd;
    const int64_t M = pl.M, d_out = pl.d_out;
    char *ws = static_cast<char *>(workspace);
    _Float16 *al = reinterpret_cast<_Float16 *>(ws + pl.off_al);
    float *a = reinterpret_cast<float *>(ws + pb.off_a);
    hipError_t e;
    // a = f16(x.g) . S_V [M][r] in f32, and al = f16(l.a) [M][kpad2] as the forward's GEMM1 writes it
    e = gemm1(pl, bits_v, l, g, x, al, a, ws, s);
    if (e != hipSuccess) return e;
    // c = al . S_U^T (not stored): partial sums of dy.c, and dyh = f16(dy.h.gs) [M][kpado] (perm4 order)
    {
        GemmArgs p = gemm2_args(pl, bits_u, al);
        p.N = (int)pb.kpado, p.nrowf = (int)d_out, p.rowf = h;
        p.ea = dy, p.ldea = d_out, p.part = reinterpret_cast<float *>(ws + pb.off_part_dh);
        p.Ch = reinterpret_cast<_Float16 *>(ws + pb.off_dyh), p.ldch = pb.kpado, p.gs = gs;
        e = gemm_short_k<kEpiBwdC>(p, s);
        if (e != hipSuccess) return e;
    }
    return backward_tail(pb, bits_u, bits_v, l, g, x, a, dx, dh, dl, dg, gs, ws, accumulate_dx,
                         blr_small_tiles(M, pl.kpad2), s);
}

// The backward from the forward's saved a [M][r] and c [M][d_out] (f32, as the
// forward computed them): the dy.c sums and dyh in one pass over dy and c, then
// the same db, dx' and finish launches, so four launches instead of five and no
// recomputation; the bits are those of the recomputing backward.
hipError_t launch_blr_backward_saved(const BlrBwdPlan &pb, const uint32_t *bits_u, const uint32_t *bits_v,
                                     const float *h, const float *l, const float *g, const float *x, const float *dy,
                                     const float *a, const float *c, float *dx, float *dh, float *dl, float *dg,
                                     float gs, void *workspace, bool accumulate_dx, hipStream_t s) {
    const BlrPlan &pl = pb.fwd;
    char *ws = static_cast<char *>(workspace);
    DycArgs q{};
    q.dy = dy, q.c = c, q.h = h;
    q.dyh = reinterpret_cast<_Float16 *>(ws + pb.off_dyh);
    q.part = reinterpret_cast<float *>(ws + pb.off_part_dh);
    q.M = pl.M, q.d_out = pl.d_out, q.N = pb.kpado, q.ldh = pb.kpado, q.blocks = pb.blocks, q.gs = gs;
    // four columns per thread when rows of dy and c are 16-byte aligned
    const bool vec = pl.d_out % 4 == 0 && ((reinterpret_cast<uintptr_t>(dy) | reinterpret_cast<uintptr_t>(c) |
                                             reinterpret_cast<uintptr_t>(h)) & 15) == 0;
    const int64_t threads = 2 * pb.blocks * (pb.kpado / (vec ? 4 : 1));
    const unsigned wgs = (unsigned)((threads + 255) / 256);
    if (vec)
        blr_dyc_kernel<4><<<dim3(wgs), dim3(256), 0, s>>>(q);
    else
        blr_dyc_kernel<1><<<dim3(wgs), dim3(256), 0, s>>>(q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return backward_tail(pb, bits_u, bits_v, l, g, x, a, dx, dh, dl, dg, gs, ws, accumulate_dx,
                         blr_small_tiles(pl.M, pl.kpad2), s);
}

}  // namespace tq2
