// Internal declarations shared by the HIP kernel files and the C-ABI layer;
// the device weight layout is described in layout.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace tq2 {

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
// Compute units of the current device (256 if the query fails), cached per device.
int device_cus();

// Skinny MFMA kernels: for K % 1024 == 0 up to kSkinny16MaxM rows (x held two
// steps at a time), otherwise up to kSkinnyMaxM rows whose x (as f16) fits in LDS.
constexpr int64_t kSkinnyMaxM = 16;
constexpr int64_t kSkinny16MaxM = 32;
constexpr size_t kSkinnyMaxLds = 160 * 1024;  // all of gfx950's LDS per workgroup
bool skinny_fits(const DevWeight &w, int64_t M);
hipError_t launch_skinny(const DevWeight &w, const float *x, float *y, int64_t M, int dev, hipStream_t s);

// Binary low-rank forward.  Workspace carve-up is computed by blr_plan: the
// f16 operand f16(l.a) [M][kpad2] that GEMM1 writes and GEMM2 reads, and, when
// GEMM1's contraction is split over ksplit1 workgroups per tile, their partial
// products [ksplit1][M][kpad2] (f32).
struct BlrPlan {
    int64_t M, d_in, d_out, r;
    int64_t kpad1, kpad2;        // contraction lengths of GEMM1 (d_in, padded) and GEMM2 (r, padded)
    int64_t ksplit1;             // GEMM1's workgroups per output tile along d_in (1: not split)
    size_t off_al, off_part1, total;
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

// accumulate: y = f32(y + f32(h*c)) instead of y = f32(h*c) (later paths of a layer);
// save_a / save_c (both or neither): also keep a [M][r] and c [M][d_out] in f32
hipError_t launch_blr_forward(const BlrPlan &p, const uint32_t *bits_u, const uint32_t *bits_v,
                              const float *h, const float *l, const float *g, const float *x, float *y,
                              void *workspace, bool accumulate, float *save_a, float *save_c, hipStream_t s);
// the backward from a forward's saved a and c (no recomputation; the same bits)
hipError_t launch_blr_backward_saved(const BlrBwdPlan &p, const uint32_t *bits_u, const uint32_t *bits_v,
                                     const float *h, const float *l, const float *g, const float *x, const float *dy,
                                     const float *a, const float *c, float *dx, float *dh, float *dl, float *dg,
                                     float gs, void *workspace, bool accumulate_dx, hipStream_t s);

}  // namespace tq2
