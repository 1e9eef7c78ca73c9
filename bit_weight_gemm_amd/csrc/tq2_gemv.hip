// Decode kernel and the f32 small-M product for TQ2_0_g128 weights (gfx950).
//
// Format ("oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs", correctness test):
// w[n][k] = (code - 1) * d with the block's f16 scale d; product
// y[m][n] = sum_k x[m][k] * w[n][k], row-major [M][N].
#include <hip/hip_runtime.h>

#include "decode.h"
#include "internal.h"

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

namespace tq2 {

// ------------------------------------------------------------------ decode

// One thread per 16-element group: w_out[n][16g + e] = (float)(q - 1) * (float)d.
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *__restrict__ codes,
                                                      const uint16_t *__restrict__ scales,
                                                      float *__restrict__ out, int64_t N, int64_t K) {
    const int64_t kw = K / 16;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= N * kw) return;
    const int64_t n = gid / kw, g = gid % kw;
    const uint32_t w = codes[code_index(n, g, kw)];
    const float d = (float)__builtin_bit_cast(_Float16, scales[scale_index(n, (g * 16) / kBlock, K / kBlock)]);
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int q = (w >> (2 * (e >> 1) + 16 * (e & 1))) & 3;
        v[e] = (float)(q - 1) * d;
    }
    f4 *o = reinterpret_cast<f4 *>(out + n * K + g * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
}

hipError_t launch_dequant(const DevWeight &w, float *out, hipStream_t s) {
    const int64_t total = w.N * (w.K / 16);
    const int64_t blocks = (total + 255) / 256;
    dequant_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(w.codes, w.scales, out, w.N, w.K);
    return hipGetLastError();
}

// ------------------------------------------------------------------ f32 small-M product
//
// Work split: a workgroup of 4 waves owns RW weight rows and MT activation rows.
// K is walked in passes of 4096: wave w takes elements [1024w, 1024w+1024) of
// the pass and lane l the 16-element group l of that range, so one wave-wide load
// reads 256 contiguous bytes of a row.  Each lane keeps its 16 x values per
// activation row in registers and, for each weight row, decodes the group word
// into 8 exact f16 pairs of (q - 1) and accumulates x*(q-1) with mixed
// f32 x f16 -> f32 fused multiply-adds (16 terms of one block), scales the partial
// by the block's d and keeps a per-lane running sum.
//
// Reduction of the RW lane sums over the wave without LDS: a lane-half exchange
// (v_permlane32_swap) adds rows r and r+RW/2 pairwise so each half of the wave
// keeps half the rows, a 16-lane-row exchange (v_permlane16_swap) halves them
// again, and DPP adds finish each 16-lane row; every row's wave sum then sits in
// one lane per 16-lane row.  The 4 waves are added through LDS.  The order of all
// additions is fixed, so results are bitwise reproducible.
template <int RW, int MT>
__global__ __launch_bounds__(256) void gemv_f32_kernel(const uint32_t *__restrict__ codes,
                                                       const uint16_t *__restrict__ scales,
                                                       const float *__restrict__ x, float *__restrict__ y,
                                                       int M, int N, int K) {
    static_assert(RW == 4 || RW == 8 || RW == 16, "rows per workgroup");
    constexpr int H1 = RW / 2, H2 = RW / 4;
    __shared__ float red[4][RW][MT];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * RW;
    const int m0 = blockIdx.y * MT;
    const int kw = K >> 4, kb = K / kBlock;
    const uint32_t magic = f16_magic();

    float acc[RW][MT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.0f;

    for (int kp = 0;;) {  // K >= 128: the first pass always runs (see gemv_mt_kernel)
        const int g = (kp >> 4) + wave * 64 + lane;  // group index within the row
        if (g < kw) {
            // Issue every load of this pass before any arithmetic, so the whole
            // pass costs one memory round trip.
            // 16-byte loads of four rows' words and 8-byte loads of their scales
            uint32_t cw[RW];
            uint16_t db[RW];
            const u4 *c4 = reinterpret_cast<const u4 *>(codes);
            const uint2 *s4 = reinterpret_cast<const uint2 *>(scales);
#pragma unroll
            for (int i = 0; i < RW / 4; ++i) {
                const u4 v = c4[(int64_t)((n0 >> 2) + i) * kw + g];
                cw[4 * i] = v.x, cw[4 * i + 1] = v.y, cw[4 * i + 2] = v.z, cw[4 * i + 3] = v.w;
            }
#pragma unroll
            for (int i = 0; i < RW / 4; ++i) {
                const uint2 v = s4[(int64_t)((n0 >> 2) + i) * kb + (g >> 3)];
                db[4 * i] = (uint16_t)(v.x & 0xFFFFu), db[4 * i + 1] = (uint16_t)(v.x >> 16);
                db[4 * i + 2] = (uint16_t)(v.y & 0xFFFFu), db[4 * i + 3] = (uint16_t)(v.y >> 16);
            }
            f4 xr[MT][4];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const f4 *xp = reinterpret_cast<const f4 *>(x + (int64_t)(m0 + t < M ? m0 + t : m0) * K + g * 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) xr[t][i] = xp[i];
            }
            __builtin_amdgcn_sched_barrier(0);
            float d[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) d[r] = (float)__builtin_bit_cast(_Float16, db[r]);
            float xv[MT][16];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool live = m0 + t < M;
                    xv[t][4 * i] = live ? xr[t][i].x : 0.0f;
                    xv[t][4 * i + 1] = live ? xr[t][i].y : 0.0f;
                    xv[t][4 * i + 2] = live ? xr[t][i].z : 0.0f;
                    xv[t][4 * i + 3] = live ? xr[t][i].w : 0.0f;
                }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                h2 p[8];
                word_m1(cw[r], magic, p);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    float s = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        s = __builtin_fmaf(xv[t][2 * i], (float)p[i].x, s);
                        s = __builtin_fmaf(xv[t][2 * i + 1], (float)p[i].y, s);
                    }
                    acc[r][t] = __builtin_fmaf(s, d[r], acc[r][t]);
                }
            }
        }
        kp += 4096;
        if (kp >= K) break;
    }

    const int k32 = kept32(), k16 = kept16();
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        float s1[H1];
#pragma unroll
        for (int r = 0; r < H1; ++r) {
            float a = acc[r][t], b = acc[r + H1][t];
            swap32(a, b);
            s1[r] = a + b;  // row r + H1*k32
        }
#pragma unroll
        for (int r = 0; r < H2; ++r) {
            float a = s1[r], b = s1[r + H2];
            swap16(a, b);
            const float v = row16_sum(a + b);  // row r + H2*k16 + H1*k32
            if ((lane & 15) == 0) red[wave][r + H2 * k16 + H1 * k32][t] = v;
        }
    }
    __syncthreads();
    if (threadIdx.x < RW * MT) {
        const int r = threadIdx.x / MT, t = threadIdx.x % MT;
        const float v = (red[0][r][t] + red[1][r][t]) + (red[2][r][t] + red[3][r][t]);
        if (n0 + r < N && m0 + t < M) y[(int64_t)(m0 + t) * N + n0 + r] = v;
    }
}

// ------------------------------------------------------------------ 1 <= M <= 4 (decode)
//
// The same per-lane work as gemv_f32_kernel<4, MT> (one 16-element group of four
// weight rows per lane and 4096-wide pass, the same f16-pair decode, fused
// multiply-adds, block scale, lane-sum exchanges and wave order of the final
// sum, so the same bits), for all MT = M <= 4 activation rows at once, with
// Q row quads per workgroup: waves 4q .. 4q+3 take row quad q.  Workgroups of
// eight waves (Q = 2) halve the workgroup count at the same wave count; the cold
// 4096 x 4096 decode takes 3.97 us against 4.09 with four-wave workgroups, and
// 3.70-3.75 us with the code words and scales, which one call reads once, loaded
// non-temporally.  Scalar base addresses, the decode's constants in scalar
// registers (word_m1_s) and the four rows' multiply-add chains interleaved take
// it from 3.63 to 3.58 us.
template <int Q, int MT>
__global__ __launch_bounds__(256 * Q) void gemv_mt_kernel(const uint32_t *__restrict__ codes,
                                                          const uint16_t *__restrict__ scales,
                                                          const float *__restrict__ x, float *__restrict__ y, int N,
                                                          int K) {
    __shared__ float red[4 * Q][4][MT];
    // the wave index is the same on every lane: read it into a scalar register,
    // so the row and group offsets below are scalar arithmetic and each load
    // adds only the lane's 32-bit offset to a scalar base
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int quad = wave >> 2, kwave = wave & 3;
    const int row0 = blockIdx.x * 4 * Q;  // first weight row of the workgroup
    const int n0 = row0 + 4 * quad;       // this wave's row quad (< Npad: padded rows are code 1)
    const int kw = K >> 4, kb = K / kBlock;
    const uint32_t magic = f16_magic();
    // the row quad's code words and scales from scalar base addresses; each
    // lane adds a 32-bit offset
    const char *cq = reinterpret_cast<const char *>(codes) + (int64_t)(n0 >> 2) * kw * 16;
    const char *sq = reinterpret_cast<const char *>(scales) + (int64_t)(n0 >> 2) * kb * 8;

    float acc[4][MT];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.0f;
    // K >= 128 (checked at upload): the first pass always runs, so the kernel
    // reads all its arguments in one scalar load instead of testing K first
    for (int kp = 0;;) {
        const int g = (kp >> 4) + kwave * 64 + lane;  // group index within the row
        if (g < kw) {
            // all loads of the pass before any arithmetic: one memory round trip; the
            // code words and scales are read once per call, so they are loaded
            // non-temporally (x, which every workgroup reads, is not)
            const u4 cv = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(cq + (uint32_t)g * 16u));
            const u2 sv = __builtin_nontemporal_load(reinterpret_cast<const u2 *>(sq + (uint32_t)(g >> 3) * 8u));
            f4 xr[MT][4];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const f4 *xp = reinterpret_cast<const f4 *>(reinterpret_cast<const char *>(x + (int64_t)t * K) +
                                                            (uint32_t)g * 64u);
#pragma unroll
                for (int i = 0; i < 4; ++i) xr[t][i] = xp[i];
            }
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
            const uint16_t db[4] = {(uint16_t)(sv.x & 0xFFFFu), (uint16_t)(sv.x >> 16), (uint16_t)(sv.y & 0xFFFFu),
                                    (uint16_t)(sv.y >> 16)};
            float xv[MT][16];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xv[t][4 * i] = xr[t][i].x, xv[t][4 * i + 1] = xr[t][i].y;
                    xv[t][4 * i + 2] = xr[t][i].z, xv[t][4 * i + 3] = xr[t][i].w;
                }
            // the four rows' sums advance together (four independent chains of
            // multiply-adds), each in the order k = 0 .. 15
            h2 p[4][8];
#pragma unroll
            for (int r = 0; r < 4; ++r) word_m1_s(cw[r], magic, p[r]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) s[r] = __builtin_fmaf(xv[t][2 * i], (float)p[r][i].x, s[r]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) s[r] = __builtin_fmaf(xv[t][2 * i + 1], (float)p[r][i].y, s[r]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r][t] = __builtin_fmaf(s[r], (float)__builtin_bit_cast(_Float16, db[r]), acc[r][t]);
            }
        }
        kp += 4096;
        if (kp >= K) break;
    }
    // per activation row: rows r and r+2 pairwise across the lane halves, then
    // across 16-lane rows, then DPP within each 16-lane row: row k16 + 2*k32's
    // wave sum in lane 16*j
    const int k32 = kept32(), k16 = kept16();
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        float s1[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            float a = acc[r][t], b = acc[r + 2][t];
            swap32(a, b);
            s1[r] = a + b;
        }
        float a = s1[0], b = s1[1];
        swap16(a, b);
        const float v = row16_sum(a + b);
        if ((lane & 15) == 0) red[wave][k16 + 2 * k32][t] = v;
    }
    __syncthreads();
    if (threadIdx.x < 4 * Q * MT) {
        const int q = threadIdx.x / (4 * MT), r = (threadIdx.x / MT) % 4, t = threadIdx.x % MT;
        const float out = (red[4 * q][r][t] + red[4 * q + 1][r][t]) + (red[4 * q + 2][r][t] + red[4 * q + 3][r][t]);
        if (row0 + 4 * q + r < N) y[(int64_t)t * N + row0 + 4 * q + r] = out;
    }
}

template <int RW, int MT>
static hipError_t gemv_launch(const DevWeight &w, const float *x, float *y, int64_t M, hipStream_t s) {
    const unsigned gx = (unsigned)(w.Npad / RW);
    // grid.y is limited to 65535 row tiles; larger M runs in slices.
    const int64_t slice = (int64_t)65535 * MT;
    for (int64_t m0 = 0; m0 < M; m0 += slice) {
        const int64_t mm = (M - m0 < slice) ? (M - m0) : slice;
        const unsigned gy = (unsigned)((mm + MT - 1) / MT);
        gemv_f32_kernel<RW, MT><<<dim3(gx, gy), dim3(256), 0, s>>>(w.codes, w.scales, x + m0 * w.K, y + m0 * w.N,
                                                                  (int)mm, (int)w.N, (int)w.K);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int MT>
static hipError_t gemv_mt_launch(const DevWeight &w, const float *x, float *y, hipStream_t s) {
    constexpr int Q = 2;  // Npad is a multiple of 256, so of 4*Q
    gemv_mt_kernel<Q, MT><<<dim3((unsigned)(w.Npad / (4 * Q))), dim3(256 * Q), 0, s>>>(w.codes, w.scales, x, y,
                                                                                    (int)w.N, (int)w.K);
    return hipGetLastError();
}

hipError_t launch_gemv_f32(const DevWeight &w, const float *x, float *y, int64_t M, hipStream_t s) {
    if (M == 1) return gemv_mt_launch<1>(w, x, y, s);
    // 2 <= M <= 4: every wave reads all M rows of x for its K range, so with
    // many weight rows x traffic outweighs the weight's; measured with cold
    // weights at K = 4096, four rows per lane win up to N = 4096 (M = 2, 3, 4:
    // 4.96, 6.1, 6.84 us against 5.34, 7.3, 7.4) and eight rows per lane from
    // N = 8192 (M = 2: 7.40 against 7.59 us; N = 14336: 11.0 against 11.9).
    if (M <= 4 && w.Npad <= 4096) {
        if (M == 2) return gemv_mt_launch<2>(w, x, y, s);
        if (M == 3) return gemv_mt_launch<3>(w, x, y, s);
        return gemv_mt_launch<4>(w, x, y, s);
    }
    if (M == 2) return gemv_launch<8, 2>(w, x, y, M, s);
    // more rows (M > 4 when the f32 path is forced): tiles of four activation rows
    return gemv_launch<8, 4>(w, x, y, M, s);
}

}  // namespace tq2
