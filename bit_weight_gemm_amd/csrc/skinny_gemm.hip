// Skinny MFMA product for few activation rows: y[m][n] = sum_k f16(x[m][k]) *
// (code-1)*d, the ternary GEMM of "oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs"
// on the f16 MFMA path (same operands and bound as the tiled kernel).
//
// For few rows (up to 32, or 16 with M*K <= 65536) a workgroup keeps x in LDS as f16,
// and its waves then run without barriers: each wave streams the code words of
// the workgroup's output columns over its own eighth of K straight from HBM into
// registers, several steps ahead, decodes them and issues MFMAs with A fragments
// read from LDS.  At the end the waves' partial tiles are added through LDS in
// wave order, so the result does not depend on timing.  Two kernels:
// skinny16_kernel (K a multiple of 1024) on v_mfma_f32_16x16x32_f16, each lane
// owning one, two or four adjacent output columns, whose words of one group it
// loads at once, with the block scale applied to each block's sum and x staged
// into LDS step by step; and
// skinny_kernel (other K) on v_mfma_f32_32x32x16_f16 with 32- or 64-column
// workgroups and d folded into the f16 operand.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>


#include "decode.h"
#include "internal.h"

namespace tq2 {

namespace {

struct SkinnyArgs {
    const float *x;          // [M][K] f32
    const uint32_t *codes;   // device layout (code_index)
    const uint16_t *scales;  // device layout (scale_index)
    float *y;                // [M][N]
    int M, N, K;
    int kw, kb;              // K/16, K/128
};

// x in LDS: row r at r*(K+8) halves.  K is a multiple of 128, so each row
// starts 16 bytes further round the 64 banks than the one before, and the 16
// rows read by one A-fragment access land on 16 different bank groups.
__device__ __forceinline__ int xs_row(int r, int K) { return r * (K + 8); }

// NBW: 32-column blocks per wave (and per workgroup); WK: waves, each owning
// K/WK of the contraction; D: steps of 64 k whose code words are in flight;
// U: pieces of x (4 values) each lane stages, with 64*U >= M*K/(4*WK).
template <int NBW, int WK, int D, int U>
__global__ __launch_bounds__(WK * 64) void skinny_kernel(SkinnyArgs p) {
    extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lrow = lane & 31, hk = lane >> 5;
    const int n0 = blockIdx.x * (32 * NBW);
    const uint32_t magic = f16_magic();

    // ---- this wave's K range and its code-word stream
    const int kw_wave = p.K / WK;      // k per wave, a multiple of 64
    const int nsteps = kw_wave / 64;   // a multiple of D
    const int kbeg = wave * kw_wave;
    int col[NBW];
    uint32_t cbase[NBW], sbase[NBW];  // word offsets of (col, group kbeg/16) and (col, block 0)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
        col[nb] = n0 + 32 * nb + lrow;  // < Npad: padded rows are code 1
        cbase[nb] = (uint32_t)code_index(col[nb], kbeg >> 4, p.kw);
        sbase[nb] = (uint32_t)scale_index(col[nb], 0, p.kb);
    }
    uint32_t bw[D][NBW][4];
    uint16_t dv[D][NBW];
    // step t: groups kbeg/16 + 4t .. +3 (16 words apart per step, 4 per group),
    // block (kbeg + 64t)/128 (4 scales apart per block; with K % 1024 == 512 a
    // wave's range starts half way through a block)
    auto load = [&](int slot, int t) {
        const uint32_t tc = (uint32_t)(t < nsteps ? t : nsteps - 1);  // clamped past the end
        const uint32_t blk = ((uint32_t)(kbeg >> 6) + tc) >> 1;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const uint32_t *cw = p.codes + cbase[nb] + 16 * tc;
#pragma unroll
            for (int i = 0; i < 4; ++i) bw[slot][nb][i] = cw[4 * i];
            dv[slot][nb] = p.scales[sbase[nb] + 4 * blk];
        }
    };
    // ---- stage x once: f32 -> f16 (round to nearest even), 4 values per piece.
    // Each wave stages the slice it reads, all M rows of its K range [kbeg,
    // kbeg + K/WK): M*qw pieces with qw = K/(4*WK) per row, lane l taking
    // U of them, 64 apart.  No wave reads another's slice, so the loop needs no
    // workgroup barrier, only the wave's own LDS stores, and each wave starts as
    // soon as its own x and code words are in.  The loads go out before the
    // weight stream starts and the LDS stores wait only for them (the memory
    // counter retires in issue order), so x comes from L2 while the first code
    // words are still on their way from HBM.  Slots past the end re-read the
    // lane's first piece and store nothing, which keeps the loads free of
    // branches.
    const int qw = kw_wave / 4;  // pieces per row of the slice (>= 16)
    const int total = p.M * qw;
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    f4 xv[U];
    // Each workgroup walks its slices from its own starting piece (wrapping at
    // the end), so the workgroups on one XCD do not all ask the same L2 channel
    // for the same line at once.  Piece u of this lane is (start + lane + 64u)
    // mod M*qw, tracked as (row, q) and advanced without divisions.
    const int start = (int)(((unsigned)blockIdx.x * 2053u) % (unsigned)total);
    const int s0 = (lane + start) % total;
    const int r0 = s0 / qw, q0 = s0 % qw;
    const int adv_r = (64 / qw) % p.M, adv_q = 64 % qw;
    auto next = [&](int &r, int &q) {
        q += adv_q;
        r += adv_r;
        if (q >= qw) {
            q -= qw;
            ++r;
        }
        if (r >= p.M) r -= p.M;
    };
    {
        int r = r0, q = q0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = u * 64 + lane < total;
            xv[u] = *reinterpret_cast<const f4 *>(p.x + (int64_t)(live ? r : r0) * p.K + kbeg + 4 * (live ? q : q0));
            next(r, q);
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the code-word loads
#pragma unroll
    for (int s = 0; s < D; ++s) load(s, s);
    __builtin_amdgcn_sched_barrier(0);
    {
        int r = r0, q = q0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u * 64 + lane < total) {
                const h4 h = {(_Float16)xv[u][0], (_Float16)xv[u][1], (_Float16)xv[u][2], (_Float16)xv[u][3]};
                *reinterpret_cast<h4 *>(&xs[xs_row(r, p.K) + kbeg + 4 * q]) = h;
            }
            next(r, q);
        }
    }

    f16x acc[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[nb] = f16x{};
    const int arow = lrow < p.M ? lrow : p.M - 1;  // rows past M repeat row M-1; never stored

    // the wave's own slice is in LDS once its stores are done (no barrier: the
    // code words in flight are not waited for here)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    for (int t0 = 0; t0 < nsteps; t0 += D) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const _Float16 *xa = xs + xs_row(arow, p.K) + kbeg + (t0 + s) * 64 + 8 * hk;
            h8 a[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const h8 *>(xa + 16 * j);
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const _Float16 d = __builtin_bit_cast(_Float16, dv[s][nb]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const h8 b = half_group_m1(bw[s][nb][j], hk, magic) * d;
                    acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b, acc[nb], 0, 0, 0);
                }
            }
            load(s, t0 + s + D);
        }
    }

    // ---- the waves' partial tiles added in wave order (LDS reused after the
    // barrier).  Registers 4j..4j+3 of a block hold its rows 8j..8j+7, so only the
    // first 4*ceil(M/8) registers hold rows below M: every wave leaves those in
    // LDS, then the waves share the sums, each (block, register) added over the
    // waves in wave order (the order of one wave adding the others, so the same
    // bits), and store them.
    __syncthreads();
    float *red = reinterpret_cast<float *>(xs);
    auto at = [&](int w, int nb, int r) { return ((w * NBW + nb) * 16 + r) * 64 + lane; };
    const int nreg = 4 * ((p.M + 7) / 8);  // 4 or 8 (M <= 16)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (r < nreg) red[at(wave, nb, r)] = acc[nb][r];  // wave-uniform
    __syncthreads();
    for (int it = wave; it < NBW * nreg; it += WK) {  // wave-uniform
        const int nb = it / nreg, r = it % nreg;
        float v = red[at(0, nb, r)];
#pragma unroll
        for (int w = 1; w < WK; ++w) v += red[at(w, nb, r)];
        // lane holds column lrow of the block, rows 8*(r/4) + 4*hk + r%4
        const int gm = 8 * (r >> 2) + 4 * hk + (r & 3), gn = n0 + 32 * nb + lrow;
        if (gm < p.M && gn < p.N) p.y[(int64_t)gm * p.N + gn] = v;
    }
}

// ---- the same product on v_mfma_f32_16x16x32_f16 (16-row MFMA blocks, so no rows
// are wasted when M is a multiple of 16), for up to 32 rows and K a multiple of
// 1024 (eight waves, each owning whole 128-wide blocks).
//
// Lane l = 16q + c holds MFMA row/column slot c and k octet q.  It owns the CPL
// adjacent weight rows (output columns) n0 + CPL*c + j, j < CPL: their code
// words of one 16-wide group lie side by side in the device layout, so one
// 4*CPL-byte load brings the lane all its words of a group, and one 2*CPL-byte
// load its scales of a block.  In step t (64 k of the wave's slice) the lane
// takes group 4t + q: elements 0..7 feed the step's first MFMA (MFMA k = 8q + i)
// and elements 8..15 its second, and the A fragments read x at the same k, so
// every decoded word feeds two MFMAs.  Column block j's MFMAs give the output
// columns n0 + CPL*c + j.  The operands are the exact codes q - 1; each block's
// two steps (four MFMAs per column block) accumulate from zero, and the block's
// sum is then scaled by d in f32 and added to the lane's total, so the decode
// has no per-weight scaling.
//
// x is staged step by step: a load slot holds one step's x pieces (rows 4i + q,
// i < PPS, k 4c .. 4c+3 of the step, f32), code words and scales, and the slots
// of D steps are in flight.  The loads go out step by step, x with its step's
// words, so a step waits only for its own data (the memory counter retires in
// issue order), and each step's x is rounded to f16 into LDS after the MFMAs of
// the step before.  Each wave keeps the x of two steps in LDS (the one its
// MFMAs read and the next), 16*RB rows of 64 k each, so up to 32 rows fit; it
// reads only the x it stores itself, so no barrier is needed.  With RB = 2 row
// blocks each decoded word feeds four MFMAs.  The last D steps issue no further
// loads.  At the end the waves' totals are added in wave order through LDS, as
// in skinny_kernel.
template <int CPL, int D, int PPS, int RB>
__global__ __launch_bounds__(512) void skinny16_kernel(SkinnyArgs p) {
    constexpr int WK = 8;
    constexpr int SW = (CPL + 1) / 2;  // 32-bit words holding the lane's CPL scales
    constexpr int XR = 16 * RB;        // rows of x a wave holds per step
    constexpr int XS = 72;             // halves per row: 64 k and 8 of padding (16 rows hit all banks)
    typedef uint32_t uw __attribute__((ext_vector_type(CPL)));
    typedef uint32_t us __attribute__((ext_vector_type(SW)));
    typedef uint16_t us1;
    typedef float fv __attribute__((ext_vector_type(CPL)));
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = lane & 15, q = lane >> 4;
    const int nl = blockIdx.x * (16 * CPL) + CPL * c;  // the lane's first column (< Npad)
    const uint32_t magic = f16_magic();

    // ---- this wave's K range; the lane's words of group kbeg/16 + q and scales
    // of block kbeg/128 (each step moves 4 groups = 64 bytes of words, each block
    // 4 scales = 8 bytes)
    const int kw_wave = p.K / WK;     // a multiple of 128
    const int nsteps = kw_wave / 64;  // even, a multiple of D
    const int kbeg = wave * kw_wave;
    const char *cp = reinterpret_cast<const char *>(p.codes) + code_index(nl, (kbeg >> 4) + q, p.kw) * 4;
    const char *sp = reinterpret_cast<const char *>(p.scales) + scale_index(nl, kbeg / kBlock, p.kb) * 2;
    const float *xg[PPS];  // rows past M re-read row M-1
#pragma unroll
    for (int i = 0; i < PPS; ++i) {
        const int r = 4 * i + q;
        xg[i] = p.x + (int64_t)(r < p.M ? r : p.M - 1) * p.K + kbeg + 4 * c;
    }
    uw bw[D];
    uint32_t dv[D][SW];
    f4 xv[D][PPS];
    auto load = [&](int slot, int t) {
#pragma unroll
        for (int i = 0; i < PPS; ++i) xv[slot][i] = *reinterpret_cast<const f4 *>(xg[i] + 64 * t);
        bw[slot] = *reinterpret_cast<const uw *>(cp + (uint32_t)t * 64u);
        if (slot & 1) {  // a block's scales, with its second step
            const char *sb = sp + (uint32_t)(t >> 1) * 8u;
            if constexpr (CPL == 1) {
                dv[slot][0] = *reinterpret_cast<const us1 *>(sb);
            } else {
                const us v = *reinterpret_cast<const us *>(sb);
#pragma unroll
                for (int i = 0; i < SW; ++i) dv[slot][i] = v[i];
            }
        }
    };
    // step t's x, rounded to f16 (nearest even), into the wave's LDS half t % 2.
    // Rows past M hold row M-1's values and store them at row M-1 again (the
    // same bits), so the stores need no branch: a branch would take the loads
    // that feed them in, and its wait would then count every load in flight.
    _Float16 *xw = xs + wave * (2 * XR * XS);
    int xrow_s[PPS];
#pragma unroll
    for (int i = 0; i < PPS; ++i) {
        const int r = 4 * i + q;
        xrow_s[i] = (r < p.M ? r : p.M - 1) * XS + 4 * c;
    }
    auto stage = [&](int slot, int t) {
#pragma unroll
        for (int i = 0; i < PPS; ++i) {
            const h4 h = {(_Float16)xv[slot][i][0], (_Float16)xv[slot][i][1], (_Float16)xv[slot][i][2],
                          (_Float16)xv[slot][i][3]};
            *reinterpret_cast<h4 *>(&xw[(t & 1) * (XR * XS) + xrow_s[i]]) = h;
        }
    };

    // the first D steps' loads in step order (kept so by the scheduling barriers)
#pragma unroll
    for (int s = 0; s < D; ++s) {
        load(s, s);
        __builtin_amdgcn_sched_barrier(0);
    }
    stage(0, 0);

    f4 acc[RB][CPL], blk[RB][CPL];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < CPL; ++j) acc[rb][j] = f4{}, blk[rb][j] = f4{};
    // A rows 16 rb + c; rows past M repeat row M-1 (never stored)
    int arow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = 16 * rb + c;
        arow[rb] = (r < p.M ? r : p.M - 1) * XS + 16 * q;
    }
    // step t from slot s: the MFMAs, then the next step's x into LDS, then
    // (MORE) the loads of step t + D into the slot
    auto body = [&](auto more, int s, int t) {
        const _Float16 *xh = xw + (t & 1) * (XR * XS);
        h8 a0[RB], a1[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            a0[rb] = *reinterpret_cast<const h8 *>(xh + arow[rb]);
            a1[rb] = *reinterpret_cast<const h8 *>(xh + arow[rb] + 8);
        }
        h8 b1[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            h2 pr[8];
            word_m1(bw[s][j], magic, pr);
            const h8 b0 = {pr[0].x, pr[0].y, pr[1].x, pr[1].y, pr[2].x, pr[2].y, pr[3].x, pr[3].y};
            b1[j] = h8{pr[4].x, pr[4].y, pr[5].x, pr[5].y, pr[6].x, pr[6].y, pr[7].x, pr[7].y};
            // a block's first step starts its sums from zero
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                blk[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[rb], b0, (s & 1) ? blk[rb][j] : f4{}, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                blk[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1[rb], b1[j], blk[rb][j], 0, 0, 0);
        if (s & 1) {  // the block's second step: add d * (block sum) to the total
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                // column j's scale: half j % 2 of word j / 2, taken with a shift
                const uint32_t dw = dv[s][j >> 1];
                const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)((j & 1) ? dw >> 16 : dw & 0xFFFFu));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[rb][j][i] = __builtin_fmaf(d, blk[rb][j][i], acc[rb][j][i]);
            }
        }
        if (s + 1 < D)
            stage(s + 1, t + 1);
        else if (decltype(more)::value)
            stage(0, t + 1);
        if constexpr (decltype(more)::value) load(s, t + D);
    };
    // One pass of the D slots (K = 512 D) runs as straight-line code: after a
    // loop the compiler's count of the loads in flight restarts from zero, so
    // every step would wait for all of them.  Two or four passes are unrolled
    // too: at a loop's entry the compiler copies the prefetched registers into
    // the loop's own, and each copy waits for its load, so the first step would
    // start only once all D steps had arrived (cold weights, K = 4096, N = 14336:
    // M = 8 8.37 -> 7.98 us, M = 16 10.34 -> 9.78, M = 32 13.64 -> 13.23; N = 4096,
    // M = 32 9.98 -> 8.65).  With one column per lane and one row block the loop
    // stays (N = 4096, M = 12 and 16 were 0.1-0.26 us slower unrolled).
    constexpr bool UNROLL = CPL >= 2 || RB == 2;
    if (nsteps == D) {
#pragma unroll
        for (int s = 0; s < D; ++s) body(std::false_type{}, s, s);
    } else if (UNROLL && nsteps == 2 * D) {
#pragma unroll
        for (int s = 0; s < D; ++s) body(std::true_type{}, s, s);
#pragma unroll
        for (int s = 0; s < D; ++s) body(std::false_type{}, s, D + s);
    } else if (UNROLL && nsteps == 4 * D) {
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
            for (int s = 0; s < D; ++s) body(std::true_type{}, s, u * D + s);
#pragma unroll
        for (int s = 0; s < D; ++s) body(std::false_type{}, s, 3 * D + s);
    } else {
        int t0 = 0;
        for (; t0 + D < nsteps; t0 += D) {
#pragma unroll
            for (int s = 0; s < D; ++s) body(std::true_type{}, s, t0 + s);
        }
#pragma unroll
        for (int s = 0; s < D; ++s) body(std::false_type{}, s, t0 + s);
    }

    // ---- the waves' totals added in wave order.  Register i of row block rb
    // and column block j holds row 16 rb + 4q + i of column nl + j; every wave
    // leaves its values in LDS (the lane's CPL columns side by side), then wave
    // w adds (rb, i) = (w / 4, w % 4) over the waves and stores the row's CPL
    // columns.
    __syncthreads();
    fv *red = reinterpret_cast<fv *>(xs);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fv v;
#pragma unroll
            for (int j = 0; j < CPL; ++j) v[j] = acc[rb][j][i];
            red[(wave * 4 * RB + 4 * rb + i) * 64 + lane] = v;
        }
    __syncthreads();
    if (wave < 4 * RB) {
        const int row = 16 * (wave >> 2) + 4 * q + (wave & 3);
        fv v = red[wave * 64 + lane];
#pragma unroll
        for (int w = 1; w < WK; ++w) v += red[(w * 4 * RB + wave) * 64 + lane];
        if (row < p.M) {
            float *yr = p.y + (int64_t)row * p.N;
            if (p.N % CPL == 0 && nl + CPL <= p.N) {
                *reinterpret_cast<fv *>(yr + nl) = v;
            } else {
#pragma unroll
                for (int j = 0; j < CPL; ++j)
                    if (nl + j < p.N) yr[nl + j] = v[j];
            }
        }
    }
}

template <int NBW, int WK, int D, int U>
hipError_t run_skinny(const SkinnyArgs &a, size_t lds, int dev, hipStream_t s) {
    // raise the kernel's dynamic LDS limit once per device (bit dev of the mask)
    static std::atomic<uint64_t> attr_set{0};
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (!bit || !(attr_set.load() & bit)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&skinny_kernel<NBW, WK, D, U>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkinnyMaxLds);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit);
    }
    const unsigned blocks = (unsigned)((a.N + 32 * NBW - 1) / (32 * NBW));
    skinny_kernel<NBW, WK, D, U><<<dim3(blocks), dim3(WK * 64), lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool skinny_fits(const DevWeight &w, int64_t M) {
    if (M < 1) return false;
    // skinny16_kernel (K % 1024 == 0; x held two steps at a time): up to 32 rows
    // at any N and K.  Measured with cold weights at K = 4096, N = 14336, M = 9..16
    // took 10.9-11.7 us (x staged whole) against the tiled kernel's 13.4.
    if (w.K % 1024 == 0) return M <= kSkinny16MaxM;
    // skinny_kernel: eight waves of 64 k-wide steps (K % 512 == 0); x staged in
    // one round of at most 32 pieces per thread (M*K/4 <= 512*32) and, as f16
    // with padded rows, within the LDS of a workgroup; more than 16 pieces per
    // thread only with 32-column workgroups (N <= 8192), where M = 12..16 took
    // 10.1-10.3 us against the tiled kernel's 13.1 at N = 4096, but 14.3 against
    // 13.7-13.8 at N = 14336.
    if (M > kSkinnyMaxM || w.K % 512 != 0 || M * w.K > 4 * 512 * 32 || (size_t)M * (w.K + 8) * 2 > kSkinnyMaxLds)
        return false;
    return M * w.K <= 4 * 512 * 16 || (w.N + 31) / 32 <= 256;
}

// Pieces of x per thread: 2, 16 or 32 (the fewest that cover M*K/4 over 512
// threads); 32 only with one column block (skinny_fits).
template <int NBW, int D>
hipError_t run_skinny_u(const SkinnyArgs &a, size_t lds, int dev, hipStream_t s) {
    const int64_t per_thread = ((int64_t)a.M * a.K / 4 + 511) / 512;
    if (per_thread <= 2) return run_skinny<NBW, 8, D, 2>(a, lds, dev, s);
    if constexpr (NBW == 1) {
        if (per_thread > 16) return run_skinny<1, 8, D, 32>(a, lds, dev, s);
    }
    return run_skinny<NBW, 8, D, 16>(a, lds, dev, s);
}

template <int CPL, int D, int PPS, int RB>
hipError_t run_skinny16(const SkinnyArgs &a, int dev, hipStream_t s) {
    static std::atomic<uint64_t> attr_set{0};
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (!bit || !(attr_set.load() & bit)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&skinny16_kernel<CPL, D, PPS, RB>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkinnyMaxLds);
        if (e != hipSuccess) return e;
        attr_set.fetch_or(bit);
    }
    // LDS: each wave's two steps of x (16 RB rows of 72 halves), later the eight
    // waves' 4 RB rows of CPL columns
    const size_t xb = (size_t)8 * 2 * 16 * RB * 72 * 2, rb = (size_t)8 * 4 * RB * 64 * CPL * 4;
    const size_t lds = xb > rb ? xb : rb;
    const unsigned blocks = (unsigned)((a.N + 16 * CPL - 1) / (16 * CPL));
    skinny16_kernel<CPL, D, PPS, RB><<<dim3(blocks), dim3(512), lds, s>>>(a);
    return hipGetLastError();
}

// x pieces per lane and step: ceil(M/4) (the rows 4i + q, i < PPS), rounded up
// to 6 or 8 past 16 rows (two row blocks).  Steps in flight: at most four from
// five rows on and with four columns per lane, and two with two row blocks,
// where more spill registers or measured slower (cold weights, K = 4096:
// N = 14336, M = 1 and 4 7.5 -> 7.0 and 7.9 -> 7.1 us with four instead of
// eight, M = 5 7.8 against 8.1; M = 8 at N = 4096 5.07 -> 4.91, at N = 6000
// 6.25 -> 6.14); up to four rows with one or two columns per lane keep eight
// (N = 4096, M = 1: 3.95 against 4.25 us with four).
template <int CPL, int D>
hipError_t run_skinny16_x(const SkinnyArgs &a, int dev, hipStream_t s) {
    constexpr int D4 = D == 8 ? 4 : D;
    if (a.M <= 4) return run_skinny16<CPL, CPL == 4 ? D4 : D, 1, 1>(a, dev, s);
    if (a.M <= 8) return run_skinny16<CPL, D4, 2, 1>(a, dev, s);
    if (a.M <= 12) return run_skinny16<CPL, D4, 3, 1>(a, dev, s);
    if (a.M <= 16) return run_skinny16<CPL, D4, 4, 1>(a, dev, s);
    if (a.M <= 24) return run_skinny16<CPL, 2, 6, 2>(a, dev, s);
    return run_skinny16<CPL, 2, 8, 2>(a, dev, s);
}

template <int CPL>
hipError_t run_skinny16_d(const SkinnyArgs &a, int dev, hipStream_t s) {
    const int steps = a.K / 512;  // per wave: even
    if (steps % 8 == 0) return run_skinny16_x<CPL, 8>(a, dev, s);
    if (steps % 4 == 0) return run_skinny16_x<CPL, 4>(a, dev, s);
    return run_skinny16_x<CPL, 2>(a, dev, s);
}

// Columns per lane of skinny16_kernel: the fewest (1, 2 or 4) that keep the
// workgroups within one round of one per CU, since a second round costs about
// as much as the first; past 4 * 16 * CUs columns, four.  More columns per lane
// mean fewer workgroups, each streaming more code words, but every workgroup
// stages all of x, so more workgroups than CUs add x traffic and a round.
// Measured with cold weights at K = 4096 (us; in brackets the earlier rule,
// the widest with at least 192 workgroups): N = 9000, M = 8 7.6 (10.65, two
// columns per lane, 282 workgroups), M = 32 12.7 (19.9); N = 5000, M = 16 8.0
// (11.1, one column per lane, 313 workgroups).  An earlier form of the kernel
// (x staged all at once) took 10.3 us at M = 8, N = 14336 with four columns per
// lane (224 workgroups), 12.8 with two and 13.9 with one.
static int skinny16_columns(int64_t N) {
    const int cus = device_cus();
    for (int cpl = 1; cpl < 4; cpl *= 2)
        if ((N + 16 * cpl - 1) / (16 * cpl) <= cus) return cpl;
    return 4;
}

hipError_t launch_skinny(const DevWeight &w, const float *x, float *y, int64_t M, int dev, hipStream_t s) {
    SkinnyArgs a{};
    a.x = x;
    a.codes = w.codes;
    a.scales = w.scales;
    a.y = y;
    a.M = (int)M;
    a.N = (int)w.N;
    a.K = (int)w.K;
    a.kw = (int)(w.K / 16);
    a.kb = (int)(w.K / kBlock);
    if (w.K % 1024 == 0) {
        const int cpl = skinny16_columns(w.N);
        if (cpl == 4) return run_skinny16_d<4>(a, dev, s);
        if (cpl == 2) return run_skinny16_d<2>(a, dev, s);
        return run_skinny16_d<1>(a, dev, s);
    }
    // Eight waves; wave w owns K/8, i.e. K/512 steps, in a multiple of the
    // prefetch depth D.  LDS: x as f16 (padded rows), later the waves' sums.
    const size_t xb = (size_t)M * (w.K + 8) * 2, rb = (size_t)8 * 16 * 64 * 4;
    const size_t lds = xb > rb ? xb : rb;
    const int64_t steps = w.K / 512;
    // one workgroup per CU: 64 columns per workgroup once 32-column ones would
    // outnumber the CUs
    if ((w.N + 31) / 32 > 256) {
        const size_t lds2 = xb > 2 * rb ? xb : 2 * rb;
        if (steps % 4 == 0) return run_skinny_u<2, 4>(a, lds2, dev, s);
        if (steps % 2 == 0) return run_skinny_u<2, 2>(a, lds2, dev, s);
        return run_skinny_u<2, 1>(a, lds2, dev, s);
    }
    if (steps % 8 == 0) return run_skinny_u<1, 8>(a, lds, dev, s);
    if (steps % 4 == 0) return run_skinny_u<1, 4>(a, lds, dev, s);
    if (steps % 2 == 0) return run_skinny_u<1, 2>(a, lds, dev, s);
    return run_skinny_u<1, 1>(a, lds, dev, s);
}

}  // namespace tq2
