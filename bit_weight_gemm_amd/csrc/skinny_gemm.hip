// Skinny MFMA product for few activation rows: y[m][n] = sum_k f16(x[m][k]) *
// (code-1)*d, the ternary GEMM of "oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs"
// on the f16 MFMA path (same operands and bound as the tiled kernel).
//
// For M <= 16 (M*K <= 65536) the whole of x fits in LDS as f16, so a workgroup stages it once
// and its waves then run without barriers: each wave streams the code words of
// the workgroup's 32 output columns over its own share of K (a half, quarter or
// eighth) straight from HBM into registers, several steps ahead, decodes them and issues
// v_mfma_f32_32x32x16_f16 with A fragments read from LDS.  At the end the waves'
// partial tiles are added through LDS in wave order, so the result does not
// depend on timing.  Workgroups are N/32, so every CU takes part even when N is
// a few thousand.
#include <hip/hip_runtime.h>

#include <atomic>

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
    uint32_t cbase[NBW], sbase[NBW];  // word offsets of (col, group kbeg/16) and (col, block kbeg/128)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
        col[nb] = n0 + 32 * nb + lrow;  // < Npad: padded rows are code 1
        cbase[nb] = (uint32_t)code_index(col[nb], kbeg >> 4, p.kw);
        sbase[nb] = (uint32_t)scale_index(col[nb], kbeg / kBlock, p.kb);
    }
    uint32_t bw[D][NBW][4];
    uint16_t dv[D][NBW];
    // step t: groups kbeg/16 + 4t .. +3 (16 words apart per step, 4 per group),
    // block kbeg/128 + t/2 (4 scales apart per block)
    auto load = [&](int slot, int t) {
        const uint32_t tc = (uint32_t)(t < nsteps ? t : nsteps - 1);  // clamped past the end
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const uint32_t *cw = p.codes + cbase[nb] + 16 * tc;
#pragma unroll
            for (int i = 0; i < 4; ++i) bw[slot][nb][i] = cw[4 * i];
            dv[slot][nb] = p.scales[sbase[nb] + 4 * (tc >> 1)];
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
    // eight waves of 64 k-wide steps: K % 512 == 0; x staged in one round of at
    // most 32 pieces per thread (M*K/4 <= 512*32) and, as f16 with padded rows,
    // within the LDS of a workgroup
    if (M < 1 || M > kSkinnyMaxM || w.K % 512 != 0 || M * w.K > 4 * 512 * 32 ||
        (size_t)M * (w.K + 8) * 2 > kSkinnyMaxLds)
        return false;
    // More than 16 pieces per thread only with 32-column workgroups (N <= 8192):
    // measured with cold weights at K = 4096, M = 12..16, the skinny kernel takes
    // 10.1-10.3 us against the tiled kernel's 13.1 at N = 4096, but 14.3 against
    // 13.7-13.8 at N = 14336 (64-column workgroups, each staging all of x).
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
