// Internal declarations shared by the HIP kernel files and the C-ABI layer.
//
// Device weight layout (built by tq2_upload from the array-of-structs blocks):
//   codes  : u32 [Npad/4][K/16][4]   one word per 16 consecutive elements of a row;
//            the words of rows 4i..4i+3 for the same 16-element group g are
//            adjacent (16 bytes), so one 16-byte load fetches a group of four rows.
//            Element e (0..15) of a group sits in bits 2*(e>>1) + 16*(e&1): even
//            elements fill the low half, odd elements the high half, each as the
//            2-bit code of the block format.  A word thus yields element pairs
//            (2s, 2s+1) as the two halves of one 32-bit register, the shape both
//            the f32 path (one pair per decode) and the MFMA operand (consecutive
//            k in the low/high halves) consume.
//   scales : u16 [Npad/4][K/128][4]  f16 bit pattern of each block's d, four rows
//            per 8-byte unit in the same row grouping.
//   Rows n >= N up to Npad (a multiple of kRowPad) hold code 1 and scale 0.
//   Word (n, g) lives at codes[((n/4) * (K/16) + g) * 4 + n%4]; scale (n, b) at
//   scales[((n/4) * (K/128) + b) * 4 + n%4].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq2 {

constexpr int kBlock = 128;      // weights per block
constexpr int kRowPad = 256;     // device rows are padded to a multiple of this

// Index of word (n, g) / scale (n, b) in the interleaved planes.
__host__ __device__ inline int64_t code_index(int64_t n, int64_t g, int64_t kw) { return ((n >> 2) * kw + g) * 4 + (n & 3); }
__host__ __device__ inline int64_t scale_index(int64_t n, int64_t b, int64_t kb) { return ((n >> 2) * kb + b) * 4 + (n & 3); }

struct DevWeight {
    int64_t N = 0, K = 0, Npad = 0;
    uint32_t *codes = nullptr;   // [Npad/4][K/16][4]
    uint16_t *scales = nullptr;  // [Npad/4][K/128][4]
    size_t bytes = 0;
    bool mfma_ok = true;         // no code-3 weight with |2d| beyond f16
};

// Each launcher validates nothing (the C-ABI layer has) and returns the HIP status.
hipError_t launch_dequant(const DevWeight &w, float *out, hipStream_t s);
hipError_t launch_gemv_f32(const DevWeight &w, const float *x, float *y, int64_t M, hipStream_t s);

// MFMA path (any M; small M uses 64-column tiles with the K range split over
// the waves of each workgroup).
hipError_t launch_gemm_mfma(const DevWeight &w, const float *x, float *y, int64_t M, hipStream_t s);

// Skinny MFMA kernel for M <= kSkinnyMaxM whose x (as f16) fits in LDS.
constexpr int64_t kSkinnyMaxM = 16;
constexpr size_t kSkinnyMaxLds = 160 * 1024;  // all of gfx950's LDS per workgroup
bool skinny_fits(const DevWeight &w, int64_t M);
hipError_t launch_skinny(const DevWeight &w, const float *x, float *y, int64_t M, int dev, hipStream_t s);

// Binary low-rank forward.  Workspace carve-up is computed by blr_plan: the
// f16 operand f16(l.a) [M][kpad2] that GEMM1 writes and GEMM2 reads.
struct BlrPlan {
    int64_t M, d_in, d_out, r;
    int64_t kpad1, kpad2;        // contraction lengths of GEMM1 (d_in, padded) and GEMM2 (r, padded)
    size_t off_al, total;
};
BlrPlan blr_plan(int64_t M, int64_t d_in, int64_t d_out, int64_t r);
// Binary low-rank backward: the forward's carve-up, then the backward's buffers.
struct BlrBwdPlan {
    BlrPlan fwd;
    int64_t kpado;               // d_out padded: contraction length of db = (dy.h) S_U
    int64_t blocks;              // blocks of 32 tokens (rows of the column partial sums)
    size_t off_a, off_dyh, off_dbl, off_part_dh, off_part_dl, off_part_dg, total;
};
BlrBwdPlan blr_bwd_plan(int64_t M, int64_t d_in, int64_t d_out, int64_t r);
// dh, dl, dg accumulate; dx is overwritten (accumulate_dx: dx = f32(dx + f32(g.dx')))
hipError_t launch_blr_backward(const BlrBwdPlan &p, const uint32_t *bits_u, const uint32_t *bits_v, const float *h,
                               const float *l, const float *g, const float *x, const float *dy, float *dx, float *dh,
                               float *dl, float *dg, float gs, void *workspace, bool accumulate_dx, hipStream_t s);

// accumulate: y = f32(y + f32(h*c)) instead of y = f32(h*c) (later paths of a layer)
hipError_t launch_blr_forward(const BlrPlan &p, const uint32_t *bits_u, const uint32_t *bits_v,
                              const float *h, const float *l, const float *g, const float *x, float *y,
                              void *workspace, bool accumulate, hipStream_t s);

}  // namespace tq2
