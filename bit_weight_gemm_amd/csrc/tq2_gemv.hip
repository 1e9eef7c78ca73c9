// Decode kernel and the f32 small-M product for TQ2_0_g128 weights (gfx950).
//
// Format ("oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs", correctness test):
// w[n][k] = (code - 1) * d with the block's f16 scale d; product
// y[m][n] = sum_k x[m][k] * w[n][k], row-major [M][N].
#include <hip/hip_runtime.h>

#include "decode.h"
#include "internal.h"

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
    const uint32_t w = codes[n * kw + g];
    const float d = (float)__builtin_bit_cast(_Float16, scales[n * (K / kBlock) + (g * 16) / kBlock]);
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
// Work split: a workgroup of 4 waves owns RW = 16 weight rows and MT activation
// rows.  K is walked in passes of 4096: wave w takes elements [1024w, 1024w+1024)
// of the pass and lane l the 16-element group l of that range, so one wave-wide
// load reads 256 contiguous bytes of a row.  Each lane keeps its 16 x values per
// activation row in registers and, for each weight row, decodes the group word
// into 8 exact f16 pairs of (q - 1) and accumulates x*(q-1) with mixed
// f32 x f16 -> f32 fused multiply-adds (16 terms, one block), scales the partial by
// the block's d, and keeps a per-lane running sum.  The lane sums are reduced
// across the wave with cross-lane adds, then across the 4 waves through LDS.
// All additions happen in a fixed order, so results are bitwise reproducible.
constexpr int kGemvRows = 16;

template <int MT>
__global__ __launch_bounds__(256) void gemv_f32_kernel(const uint32_t *__restrict__ codes,
                                                       const uint16_t *__restrict__ scales,
                                                       const float *__restrict__ x, float *__restrict__ y,
                                                       int M, int N, int K) {
    constexpr int RW = kGemvRows;
    __shared__ float red[4][RW][MT];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * RW;
    const int m0 = blockIdx.y * MT;
    const int kw = K >> 4, kb = K / kBlock;

    float acc[RW][MT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.0f;

    for (int kp = 0; kp < K; kp += 4096) {
        const int g = (kp >> 4) + wave * 64 + lane;  // group index within the row
        if (g < kw) {
            float xv[MT][16];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (m0 + t < M) {
                    const f4 *xp = reinterpret_cast<const f4 *>(x + (int64_t)(m0 + t) * K + g * 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const f4 v = xp[i];
                        xv[t][4 * i] = v.x, xv[t][4 * i + 1] = v.y, xv[t][4 * i + 2] = v.z, xv[t][4 * i + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) xv[t][e] = 0.0f;
                }
            }
            uint32_t cw[RW];
            float d[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                cw[r] = codes[(int64_t)(n0 + r) * kw + g];
                d[r] = (float)__builtin_bit_cast(_Float16, scales[(int64_t)(n0 + r) * kb + (g >> 3)]);
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                h2 p[8];
                word_m1(cw[r], p);
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
    }

#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float v = acc[r][t];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) red[wave][r][t] = v;
        }
    __syncthreads();
    if (threadIdx.x < RW * MT) {
        const int r = threadIdx.x / MT, t = threadIdx.x % MT;
        const float v = (red[0][r][t] + red[1][r][t]) + (red[2][r][t] + red[3][r][t]);
        if (n0 + r < N && m0 + t < M) y[(int64_t)(m0 + t) * N + n0 + r] = v;
    }
}

hipError_t launch_gemv_f32(const DevWeight &w, const float *x, float *y, int64_t M, hipStream_t s) {
    const unsigned gx = (unsigned)(w.Npad / kGemvRows);
    if (M == 1) {
        gemv_f32_kernel<1><<<dim3(gx, 1), dim3(256), 0, s>>>(w.codes, w.scales, x, y, 1, (int)w.N, (int)w.K);
        return hipGetLastError();
    }
    if (M == 2) {
        gemv_f32_kernel<2><<<dim3(gx, 1), dim3(256), 0, s>>>(w.codes, w.scales, x, y, 2, (int)w.N, (int)w.K);
        return hipGetLastError();
    }
    // grid.y is limited to 65535 row tiles of 4; larger M runs in slices.
    const int64_t slice = 65535 * 4;
    for (int64_t m0 = 0; m0 < M; m0 += slice) {
        const int64_t mm = (M - m0 < slice) ? (M - m0) : slice;
        const unsigned gy = (unsigned)((mm + 3) / 4);
        gemv_f32_kernel<4><<<dim3(gx, gy), dim3(256), 0, s>>>(w.codes, w.scales, x + m0 * w.K, y + m0 * w.N,
                                                              (int)mm, (int)w.N, (int)w.K);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tq2
