// Binary low-rank layer ("cortiq-engine 0.8.43 -- train_mm.rs", module header,
// blr_forward / blr_backward): the sign bitmaps re-laid as 2-bit codes, and the
// layer's products on the block-tiled MFMA kernel of mfma_gemm.h.
#include "mfma_gemm.h"

namespace tq2 {

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

// Products with the long contraction (GEMM1 over d_in, and the backward's db over
// d_out), of M x r outputs: 32 x 64 tiles when they are few, each wave taking two
// 64-wide slices of a 512-wide step when the padded contraction allows (fewer
// steps and barriers), else 128 x 128 tiles.
template <int EPI>
static hipError_t gemm_long_k(const GemmArgs &p, int64_t kpad, bool small, hipStream_t s) {
    if (!small) return run_gemm<128, 128, 1, 4, 1, 4, kAHalf, false, EPI>(p, s);
    if (kpad % 1024 == 0) return run_gemm<32, 64, 1, 2, 4, 2, kAHalf, false, EPI, 2, 1, 2>(p, s);
    return run_gemm<32, 64, 1, 2, 4, 2, kAHalf, false, EPI>(p, s);
}
// Products with the short contraction r (GEMM2, and the backward's dx'): 64 x 128
// tiles of eight waves (two k groups), A loaded two steps ahead.
template <int EPI>
static hipError_t gemm_short_k(const GemmArgs &p, hipStream_t s) {
    return run_gemm<64, 128, 1, 4, 2, 2, kAHalf, false, EPI, 2, 2>(p, s);
}

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
// contraction index k.  A thread makes the 16-byte unit of four rows
// (4q .. 4q+3) for one 16-wide k group g.  Two orientations of the bitmap:
//   kRowBits: sign(n, k) = bit n of bits[k][n/32] (rows n are the rank: S_V in
//             the forward, S_U^T in the backward): a wave takes 64 consecutive
//             row quads of one group, so each of its 16 loads (one per k)
//             touches 8 bitmap words shared by the lanes;
//   kKBits:   sign(n, k) = bit k of bits[n][k/32] (the contraction is the rank:
//             S_U in the forward, S_V in the backward): the threads walk (row
//             quad, group) with the group fastest, so a wave's loads read whole
//             bitmap rows and its stores are contiguous.
// Out-of-range elements read a valid word and are replaced by code 1.
enum RelayKind { kRowBits = 0, kKBits = 1 };
struct RelayJob {
    const uint32_t *bits;
    uint32_t *codes;
    int64_t nvalid, kvalid;  // rows and contraction indices present (the rank is one of them)
    int64_t npad, kpad;      // padded rows and contraction of the code plane
    int64_t nblk;            // workgroups of the launch this job takes
    int kind;
};

static RelayJob relay_job(int kind, const uint32_t *bits, uint32_t *codes, int64_t nvalid, int64_t kvalid,
                          int64_t npad, int64_t kpad) {
    RelayJob j{};
    j.bits = bits, j.codes = codes, j.nvalid = nvalid, j.kvalid = kvalid, j.npad = npad, j.kpad = kpad, j.kind = kind;
    j.nblk = kind == kRowBits ? ((npad / 4 + 255) / 256) * (kpad / 16) : ((npad / 4) * (kpad / 16) + 255) / 256;
    return j;
}

// One launch: the re-layout jobs in order, then (blocks after them) xg[m][k] =
// f16(x[m][k] * g[k]) (product in f32, round to nearest even) for k < d_in and 0
// up to kpad1, 8 values per thread.
constexpr int kMaxRelayJobs = 4;
struct BlrPrep {
    RelayJob job[kMaxRelayJobs];
    int njobs;
    int64_t words;                     // r / 32
    const float *x, *g;
    _Float16 *xg;
    int64_t M, d_in, kpad1;
    int xvec;                          // x rows and g allow 16-byte loads
};

// code of element e (0..15) at its place in a group word
__device__ __forceinline__ uint32_t code_at(uint32_t code, int e) { return code << (2 * (e >> 1) + 16 * (e & 1)); }

__device__ __forceinline__ void relay_row_bits(const RelayJob &j, int64_t words, int64_t bid) {
    const int64_t kw = j.kpad / 16, quads = j.npad / 4;
    const int64_t qblocks = (quads + 255) / 256;
    const int64_t quad = (bid % qblocks) * 256 + threadIdx.x, g = bid / qblocks;
    if (quad >= quads) return;
    const int64_t n0 = quad * 4;
    const bool nin = n0 < j.nvalid;  // the rank is a multiple of 32: a quad is wholly inside or past it
    const int64_t wrd = nin ? n0 >> 5 : 0;
    const int sh = (int)(n0 & 31);
    u4 out = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int64_t k = g * 16 + e;
        const bool in = nin && k < j.kvalid;
        const uint32_t bits = (j.bits[(in ? k : 0) * words + wrd] >> sh) & 15u;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) out[rr] |= code_at(in ? (((bits >> rr) & 1u) ? 2u : 0u) : 1u, e);
    }
    *reinterpret_cast<u4 *>(j.codes + (quad * kw + g) * 4) = out;
}

__device__ __forceinline__ void relay_k_bits(const RelayJob &j, int64_t words, int64_t bid) {
    const int64_t kw = j.kpad / 16;
    const int64_t item = bid * 256 + threadIdx.x;
    if (item >= (j.npad / 4) * kw) return;
    const int64_t quad = item / kw, g = item % kw;
    u4 out;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int64_t n = quad * 4 + rr;
        const bool in = n < j.nvalid && g * 16 < j.kvalid;
        const uint32_t half = (j.bits[(in ? n : 0) * words + (in ? g >> 1 : 0)] >> (16 * (g & 1))) & 0xFFFFu;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const bool ine = in && g * 16 + e < j.kvalid;
            w |= code_at(ine ? (((half >> e) & 1u) ? 2u : 0u) : 1u, e);
        }
        out[rr] = w;
    }
    *reinterpret_cast<u4 *>(j.codes + (quad * kw + g) * 4) = out;
}

__global__ __launch_bounds__(256) void blr_prep_kernel(BlrPrep q) {
    int64_t bid = blockIdx.x;
#pragma unroll
    for (int jb = 0; jb < kMaxRelayJobs; ++jb) {
        if (jb >= q.njobs) break;
        if (bid < q.job[jb].nblk) {
            if (q.job[jb].kind == kRowBits)
                relay_row_bits(q.job[jb], q.words, bid);
            else
                relay_k_bits(q.job[jb], q.words, bid);
            return;
        }
        bid -= q.job[jb].nblk;
    }
    {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        const int64_t per_row = q.kpad1 / 8;
        const int64_t piece = bid * 256 + threadIdx.x;
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

// The forward's preparation: both bitmaps re-laid and f16(x.g), one launch.
static BlrPrep forward_prep(const BlrPlan &pl, const uint32_t *bits_u, const uint32_t *bits_v, uint32_t *codes_u,
                            uint32_t *codes_v, const float *x, const float *g, _Float16 *xg) {
    BlrPrep q{};
    q.job[0] = relay_job(kRowBits, bits_v, codes_v, pl.r, pl.d_in, pl.npad1, pl.kpad1);   // S_V
    q.job[1] = relay_job(kKBits, bits_u, codes_u, pl.d_out, pl.r, pl.npad2, pl.kpad2);    // S_U
    q.njobs = 2;
    q.words = pl.r / 32;
    q.x = x, q.g = g, q.xg = xg, q.M = pl.M, q.d_in = pl.d_in, q.kpad1 = pl.kpad1;
    q.xvec = (pl.d_in % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
             ((reinterpret_cast<uintptr_t>(g) & 15) == 0);
    return q;
}

static hipError_t run_prep(const BlrPrep &q, hipStream_t s) {
    int64_t blocks = (q.M * (q.kpad1 / 8) + 255) / 256;
    for (int j = 0; j < q.njobs; ++j) blocks += q.job[j].nblk;
    if (blocks < 1) return hipSuccess;
    blr_prep_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(q);
    return hipGetLastError();
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
        hipError_t e = run_prep(forward_prep(pl, bits_u, bits_v, codes_u, codes_v, x, g, xg), s);
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
    e = gemm_long_k<kEpiHalfScale>(p1, pl.kpad1, blr_small_tiles(pl.M, pl.kpad2), s);
    if (e != hipSuccess) return e;
    // GEMM2: c = al . S_U^T, written as y (see below)
    GemmArgs p2{};
    p2.Ah = al, p2.lda = pl.kpad2;
    p2.codes = codes_u, p2.kw = pl.kpad2 / 16, p2.scales = nullptr, p2.kbw = 0;
    p2.C = y, p2.ldc = pl.d_out, p2.rowf = h;
    p2.M = (int)pl.M, p2.N = (int)pl.d_out, p2.K = (int)pl.kpad2, p2.Kloop = (int)pl.kpad2;
    // y = h . c (later paths of a layer: y = f32(y + f32(h . c)))
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
    const size_t ch = (size_t)(p.chunks > 0 ? p.chunks : 1);
    p.off_part_dh = take(ch * d_out * 4);
    p.off_part_dl = take(ch * r * 4);
    p.off_part_dg = take(ch * d_in * 4);
    p.total = off;
    return p;
}

namespace {

enum ColMode { kColStageH = 0, kColDx = 1, kColDxAcc = 2 };

// Pass 2 of a column sum, for column n: out[n] = f32(out[n] + f32(sum over chunks
// in order of part[ch][n])).  The loads of a group of chunks are independent:
// issue them together, then add in order.
__device__ __forceinline__ void column_finish(const float *__restrict__ part, float *__restrict__ out, int64_t N,
                                              int64_t chunks, int64_t n) {
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

// Pass 1 of a column sum: part[ch][n] = sum over tokens t of chunk ch of
// A[t][n] * B[t][n] (f32, ascending t), for n < N.  Fused with the elementwise
// op that reads the same operand A:
//   kColStageH: H[t][n] = f16(A[t][n] * f[n] * gs) for n < N, 0 for N <= n < ldh;
//   kColDx:     D[t][n] = f[n] * B[t][n];
//   kColDxAcc:  D[t][n] = f32(D[t][n] + f32(f[n] * B[t][n])).
// Workgroups past the column blocks (chunk 0 only) run pass 2 of an earlier
// column sum (fpart -> fout, fN columns, fchunks chunks), which saves it a launch
// of its own; its partials are in a buffer of their own, so the two do not meet.
struct ColArgs {
    const float *A, *B, *f;
    float *part;
    _Float16 *H;
    float *D;
    int64_t M, N, lda, ldh;
    float gs;
    const float *fpart;  // earlier column sum to finish, or nullptr
    float *fout;
    int64_t fN, fchunks;
};

template <int MODE>
__global__ __launch_bounds__(256) void blr_colsum_kernel(ColArgs q) {
#pragma clang fp contract(off)
    const int64_t ncols = MODE == kColStageH ? q.ldh : q.N;
    const int64_t cblocks = (ncols + 255) / 256;
    if ((int64_t)blockIdx.x >= cblocks) {
        const int64_t n = ((int64_t)blockIdx.x - cblocks) * 256 + threadIdx.x;
        if (blockIdx.y == 0 && n < q.fN) column_finish(q.fpart, q.fout, q.fN, q.fchunks, n);
        return;
    }
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t ch = blockIdx.y;
    const int64_t t0 = ch * kColChunk, t1 = t0 + kColChunk < q.M ? t0 + kColChunk : q.M;
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

// Pass 2 alone (the last column sum of a path).
__global__ __launch_bounds__(256) void blr_colsum_finish_kernel(const float *__restrict__ part, float *__restrict__ out,
                                                                int64_t N, int64_t chunks) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n < N) column_finish(part, out, N, chunks, n);
}

// Pass 1 of q (and pass 2 of the column sum q.fpart names, if any).
template <int MODE>
hipError_t colsum_pass1(const ColArgs &q, int64_t chunks, hipStream_t s) {
    const int64_t ncols = MODE == kColStageH ? q.ldh : q.N;
    const int64_t fblocks = q.fpart ? (q.fN + 255) / 256 : 0;
    blr_colsum_kernel<MODE><<<dim3((unsigned)((ncols + 255) / 256 + fblocks), (unsigned)chunks), dim3(256), 0, s>>>(q);
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
    float *part_dh = reinterpret_cast<float *>(at(pb.off_part_dh));
    float *part_dl = reinterpret_cast<float *>(at(pb.off_part_dl));
    float *part_dg = reinterpret_cast<float *>(at(pb.off_part_dg));
    hipError_t e;
    // bitmaps in both orientations and f16(x.g), one launch
    {
        BlrPrep q = forward_prep(pl, bits_u, bits_v, codes_u, codes_v, x, g, xg);
        // S_U^T: rows r, contraction d_out (bits along the rows, as S_V's);
        // S_V: rows d_in, contraction r (bits along the contraction, as S_U's)
        q.job[2] = relay_job(kRowBits, bits_u, codes_ut, r, d_out, pl.npad1, pb.kpado);
        q.job[3] = relay_job(kKBits, bits_v, codes_vt, d_in, r, pb.npadi, pl.kpad2);
        q.njobs = 4;
        e = run_prep(q, s);
        if (e != hipSuccess) return e;
    }
    const bool small = blr_small_tiles(M, pl.kpad2);
    // a = xg . S_V [M][r] in f32, and al = f16(l.a) [M][kpad2] as the forward's GEMM1 writes it
    {
        GemmArgs p{};
        p.Ah = xg, p.lda = pl.kpad1, p.codes = codes_v, p.kw = pl.kpad1 / 16;
        p.C = a, p.ldc = r, p.Ch = al, p.ldch = pl.kpad2, p.rowf = l, p.nrowf = (int)r;
        p.M = (int)M, p.N = (int)pl.kpad2, p.K = (int)pl.kpad1, p.Kloop = (int)pl.kpad1;
        e = gemm_long_k<kEpiStoreHalf>(p, pl.kpad1, small, s);
        if (e != hipSuccess) return e;
    }
    // c = al . S_U^T   [M][d_out]
    {
        GemmArgs p{};
        p.Ah = al, p.lda = pl.kpad2, p.codes = codes_u, p.kw = pl.kpad2 / 16;
        p.C = c, p.ldc = d_out, p.M = (int)M, p.N = (int)d_out, p.K = (int)pl.kpad2, p.Kloop = (int)pl.kpad2;
        e = gemm_short_k<kEpiStore>(p, s);
        if (e != hipSuccess) return e;
    }
    // dh += sum_t dy.c, with dyh = f16(dy.h.gs) staged from the same reads
    {
        ColArgs q{};
        q.A = dy, q.B = c, q.f = h, q.part = part_dh, q.H = dyh, q.M = M, q.N = d_out, q.lda = d_out, q.ldh = pb.kpado;
        q.gs = gs;
        e = colsum_pass1<kColStageH>(q, pb.chunks, s);
        if (e != hipSuccess) return e;
    }
    // db = dyh . S_U / gs   [M][r]
    {
        GemmArgs p{};
        p.Ah = dyh, p.lda = pb.kpado, p.codes = codes_ut, p.kw = pb.kpado / 16;
        p.C = db, p.ldc = r, p.M = (int)M, p.N = (int)r, p.K = (int)pb.kpado, p.Kloop = (int)pb.kpado;
        p.alpha = 1.0f / gs;
        e = gemm_long_k<kEpiScale>(p, pb.kpado, small, s);
        if (e != hipSuccess) return e;
    }
    // dl += sum_t a.db, with dbl = f16(db.l.gs) staged from the same reads
    {
        ColArgs q{};
        q.A = db, q.B = a, q.f = l, q.part = part_dl, q.H = dbl, q.M = M, q.N = r, q.lda = r, q.ldh = pl.kpad2;
        q.gs = gs;
        q.fpart = part_dh, q.fout = dh, q.fN = d_out, q.fchunks = pb.chunks;  // and dh's second pass
        e = colsum_pass1<kColStageH>(q, pb.chunks, s);
        if (e != hipSuccess) return e;
    }
    // dx' = dbl . S_V^T / gs   [M][d_in]
    {
        GemmArgs p{};
        p.Ah = dbl, p.lda = pl.kpad2, p.codes = codes_vt, p.kw = pl.kpad2 / 16;
        p.C = dxp, p.ldc = d_in, p.M = (int)M, p.N = (int)d_in, p.K = (int)pl.kpad2, p.Kloop = (int)pl.kpad2;
        p.alpha = 1.0f / gs;
        e = gemm_short_k<kEpiScale>(p, s);
        if (e != hipSuccess) return e;
    }
    // dg += sum_t x.dx', and dx = g.dx' (later paths: dx = f32(dx + f32(g.dx')))
    {
        ColArgs q{};
        q.A = x, q.B = dxp, q.f = g, q.part = part_dg, q.D = dx, q.M = M, q.N = d_in, q.lda = d_in;
        q.fpart = part_dl, q.fout = dl, q.fN = r, q.fchunks = pb.chunks;  // and dl's second pass
        e = accumulate_dx ? colsum_pass1<kColDxAcc>(q, pb.chunks, s) : colsum_pass1<kColDx>(q, pb.chunks, s);
        if (e != hipSuccess) return e;
        blr_colsum_finish_kernel<<<dim3((unsigned)((d_in + 255) / 256)), dim3(256), 0, s>>>(part_dg, dg, d_in, pb.chunks);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tq2
