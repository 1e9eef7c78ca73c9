/*
 * libtq2 -- ternary (TQ2_0_g128) weight GEMM and binary low-rank layer forward
 * for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI: host or device pointers and sizes only.  Every device pointer
 * named below is a HIP device allocation owned by the caller (for example the
 * storage of a torch tensor on the same GPU); it must stay alive until the work
 * queued on `stream` has finished.  `stream` is a hipStream_t passed as void*;
 * NULL means the legacy default stream of the current device.  All calls act on
 * the current HIP device.
 *
 * Status codes: every entry point returns TQ2_OK (0) or a negative TQ2_E* code.
 * Argument errors are detected on the host before anything is queued and leave
 * the outputs untouched.  Launch failures return TQ2_EDEVICE.  Faults inside a
 * kernel surface, as usual for HIP, at the caller's next synchronisation.
 *
 * Sources, by page title and section:
 *  [TQ2]  "oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs": the correctness test
 *         defines the block format (128 weights per block: 32 bytes of 2-bit codes,
 *         four per byte with the first element in the low bits, then an f16
 *         scale d; codes 0,1,2 = -1,0,+1, w = (code-1)*d), the weight upload
 *         (get_or_upload_tq2_weight_soa: AoS bytes in, device handle out, free to
 *         repack) and the product encode_gemm_tq2 (out[m][n] = sum_k x[m][k]*W[n][k],
 *         row-major [M][N], overwritten).
 *  [BLR]  "cortiq-engine 0.8.43 -- train_mm.rs": the module header defines the
 *         binary low-rank layer W^ = diag(h) S_U diag(l) S_V^T diag(g) and its
 *         forward a = (x.g) S_V, c = (a.l) S_U^T, y = h.c; `expand` fixes the sign
 *         bitmap (bit j of word w is rank index 32w+j, set = +1, clear = -1);
 *         `blr_forward` overwrites y and stages x.g and a.l in f16; a layer is
 *         the sum of its paths (y = sum_p W^_p x), two paths combined by
 *         `scale_acc2` as fl(fl(h_0 c_0) + fl(h_1 c_1)); the module header also
 *         gives the backward (dh, db, dl, dx', dg, dx), and `blr_backward` its f16
 *         staging under a power-of-two gradient scale.
 */
#ifndef LIBTQ2_H
#define LIBTQ2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TQ2_OK = 0,
    TQ2_EINVAL = -1,      /* bad argument: shape, size, pointer, alignment, non-finite scale */
    TQ2_ENOMEM = -2,      /* device or host allocation failed */
    TQ2_EDEVICE = -3,     /* a HIP call or kernel launch failed */
    TQ2_ENODEV = -4,      /* no HIP device, or the current device is not gfx950 */
    TQ2_ETOOBIG = -5,     /* blr_forward_noalloc: the sizes need more than its static scratch */
};

/* Bytes of the fixed device scratch array that blr_forward_noalloc uses (per GPU). */
#define TQ2_STATIC_SCRATCH_BYTES (16u << 20)

enum {
    TQ2_PATH_AUTO = 0,    /* choose by M (see tq2_select_path) */
    TQ2_PATH_F32 = 1,     /* f32 FMA path: |err| <= 1e-5 * sum_k |x*w| per output */
    TQ2_PATH_MFMA = 2,    /* f16 MFMA path: x rounded to f16, |err| <= 4e-3 * sum_k |x*w| */
};

/* Opaque device-resident weight.  Owns its device memory until tq2_free. */
typedef struct tq2_weight tq2_weight;

/* [TQ2] weight upload.  `aos` is host memory holding N*(K/128) blocks of 34 bytes,
 * row-major over (row, block): 32 code bytes then the f16 scale, little-endian.
 * Requires 1 <= N <= 2^31 - 256, 128 <= K <= 2^30, K % 128 == 0, nbytes == N*(K/128)*34 and every scale
 * finite (a NaN or infinite scale is TQ2_EINVAL).  The bytes are repacked on the
 * host into the device layout and copied on `stream`; the call returns after the
 * copy has completed, so `aos` may be freed at once.  *out receives the handle. */
int tq2_upload(const void *aos, size_t nbytes, int64_t N, int64_t K, void *stream, tq2_weight **out);

/* Releases the handle and its device memory (synchronises the device first).
 * NULL is accepted and ignored. */
int tq2_free(tq2_weight *w);

/* Shape and device footprint of a handle (any output pointer may be NULL). */
int tq2_weight_info(const tq2_weight *w, int64_t *N, int64_t *K, size_t *device_bytes);

/* [TQ2] y[m][n] = sum_k x[m][k] * W[n][k] for m < M, n < N.
 * x: device f32 [M][K] row-major, 16-byte aligned; y: device f32 [M][N] row-major,
 * 16-byte aligned, overwritten, must not overlap x.  N and K must equal the
 * handle's.  M == 0 is a successful no-op.  Asynchronous on `stream`.
 * The path follows tq2_select_path(M).  Results are deterministic: repeated calls
 * with the same inputs give the same bits.  No device memory is allocated. */
int tq2_gemm(const tq2_weight *w, const float *x, float *y, int64_t M, int64_t N, int64_t K, void *stream);

/* tq2_gemm on an explicitly chosen path (TQ2_PATH_AUTO, _F32 or _MFMA).
 * The MFMA path rounds x to f16 (nearest even) and needs |x| <= 65504 (not
 * checked).  Its per-output bound 4e-3 * sum_k |x*w| holds when that rounding is
 * relative, i.e. every nonzero |x| >= 2^-14 (f16 normal range); smaller values
 * become f16 subnormals whose rounding error is up to 2^-25 absolute, so a row
 * of x made only of such values (|x| below ~1e-5) can miss the relative bound:
 * run those on the f32 path (or scale x by a power of two first).  A weight
 * holding a code-3 weight whose scale has |d| > 32752 (2d beyond f16) runs on
 * the f32 path. */
int tq2_gemm_path(const tq2_weight *w, const float *x, float *y, int64_t M, int64_t N, int64_t K,
                  int path, void *stream);

/* Path that TQ2_PATH_AUTO picks for a product with M rows.  The threshold is the
 * process default (tq2_set_m_small, else env TQ2_M_SMALL, else 4): M <= threshold
 * runs the f32 path.  Env TQ2_PATH=f32|mfma forces a path for every auto call. */
int tq2_select_path(int64_t M);

/* Sets the auto-path threshold (M <= m_small runs on the f32 path); returns the old one. */
int64_t tq2_set_m_small(int64_t m_small);

/* Forces the path of every TQ2_PATH_AUTO call in the process (tq2_gemm):
 * TQ2_PATH_AUTO (0) restores the choice by M, TQ2_PATH_F32 (1) or TQ2_PATH_MFMA
 * (2) forces that path (the env variable TQ2_PATH=f32|mfma sets the initial
 * value).  Returns the previous setting, or TQ2_EINVAL for another value.  The
 * page validates each kernel variant through helpers that bypass the public
 * dispatch; this is the same switch for a whole process. */
int tq2_set_path(int path);

/* [TQ2] decode on the GPU: w_out[n][k] = (code-1)*d as f32, device [N][K] row-major,
 * 16-byte aligned.  Bit-exact with the format's definition (including -0.0 for a
 * zero code under a negative scale).  Asynchronous on `stream`. */
int tq2_dequant(const tq2_weight *w, float *w_out, void *stream);

/* [BLR] y[t][i] = h[i] * sum_k f16(a[t][k]*l[k]) * S_U[i][k],
 *        a[t][k] = sum_j f16(x[t][j]*g[j]) * S_V[j][k]          (f32 accumulation).
 * bits_u: device u32 [d_out][r/32], bits_v: device u32 [d_in][r/32] (the sign
 * bitmaps, 4-byte aligned); h [d_out], l [r], g [d_in]: device f32; x: device f32
 * [M][d_in]; y: device f32 [M][d_out], overwritten, 16-byte aligned, must not
 * overlap the inputs.  Requires d_in >= 1, d_out >= 1, r >= 32, r % 32 == 0, M >= 0
 * (M == 0 is a no-op), and each bitmap with 512 more rows under 2 GB
 * ((rows + 512) * r/8 < 2^31 bytes).  The f16(a*l) intermediate (and, for sizes
 * where the first product's contraction is split over workgroups, its f32
 * partial products) lives in a workspace that the library owns: one grow-only device buffer per (device, stream), allocated on
 * first use and enlarged (never shrunk) when a call needs more, kept until the
 * process ends (tq2_workspace_allocs counts these allocations).  The page's
 * layer likewise keeps its staging buffers in a scratch object it reuses.
 * Preconditions (not checked): |x*g| and |a*l| within f16 range.
 * Asynchronous on `stream`. */
int blr_forward(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out,
                int64_t r, void *stream);

/* For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Computes exactly what
 * blr_forward computes (the same kernels, so the same bits), with its workspace
 * in a fixed device array of TQ2_STATIC_SCRATCH_BYTES (16 MiB) that the library
 * holds on each GPU it runs on from module load until the process ends; the call
 * itself allocates nothing.  Sizes whose workspace (blr_workspace_size) exceeds
 * that array return TQ2_ETOOBIG before anything is queued.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other streams,
 * other host threads) race and give wrong results; serialise them.  Nothing in
 * the array needs clearing between calls (each launch writes what it reads). */
int blr_forward_noalloc(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                        const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out,
                        int64_t r, void *stream);

/* [BLR] A layer of P paths, y = sum_p h_p . c_p, each path the product of
 * blr_forward with its own bitmaps and vectors (all paths share M, d_in, d_out
 * and r).  The sum is rounded path by path as the page's scale_acc /
 * scale_acc2 kernels round it: y = f32(h_0*c_0), then y = f32(y + f32(h_p*c_p))
 * for p = 1 .. P-1, each product rounded before the addition.  Per-path operands
 * are stacked in device memory: bits_u [P][d_out][r/32], bits_v [P][d_in][r/32],
 * h [P][d_out], l [P][r], g [P][d_in].  Requires 1 <= P <= 4096 and everything
 * blr_forward requires; the paths run one after another on `stream`, sharing
 * one path's workspace (the library's, as for blr_forward).  P == 1 gives
 * blr_forward's result. */
int blr_forward_paths(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                      const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                      void *stream);

/* Bytes of device workspace blr_forward_ws / blr_forward_paths_ws need (0 on bad sizes). */
size_t blr_workspace_size(int64_t M, int64_t d_in, int64_t d_out, int64_t r);

/* blr_forward / blr_forward_paths with a caller-owned workspace instead of the
 * library's: `workspace` is device memory of at least blr_workspace_size(...)
 * bytes, 256-byte aligned, not overlapping y; its contents are scratch.  Calls
 * sharing a workspace must not overlap in time. */
int blr_forward_ws(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                   const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out,
                   int64_t r, void *workspace, size_t workspace_bytes, void *stream);
int blr_forward_paths_ws(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                         const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                         void *workspace, size_t workspace_bytes, void *stream);

/* [BLR] Backward of blr_forward_paths on the same x, path by path (the page's
 * blr_backward; per path a = (x.g) S_V and c = (a.l) S_U^T as in the forward):
 *   dh_p += sum_t dy.c      db = (dy.h) S_U      dl_p += sum_t a.db
 *   dx'  = (db.l) S_V^T     dg_p += sum_t x.dx'  dx = sum_p g.dx'
 * The two new products stage their inputs in f16 as f16(dy.h.gscale) and
 * f16(db.l.gscale) and multiply their f32 results by 1/gscale; gscale must be a
 * power of two in (0, 65536].  a and c are recomputed with the forward's kernels.
 * Sums over tokens are f32 in a fixed order (within each block of 32 tokens in
 * a fixed order, then the blocks in order), so results are reproducible.  dh [P][d_out], dl [P][r], dg [P][d_in]
 * are accumulated (y = f32(y + s)); dx [M][d_in] is overwritten by path 0 and the
 * later paths add f32(g.dx') to it.  Operands as for blr_forward_paths, plus dy:
 * device f32 [M][d_out]; all device pointers 4-byte aligned and l 16-byte
 * aligned; outputs must not overlap each other or the inputs.
 * 1 <= P <= 4096; M == 0 is a no-op.
 * The workspace is the library's (as for blr_forward).
 * Preconditions (not checked): the forward's, and |dy.h.gscale| and |db.l.gscale|
 * within f16 range (choose gscale so that they are neither huge nor subnormal).
 * Asynchronous on `stream`. */
int blr_backward_paths(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                       const float *g, const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg,
                       int64_t M, int64_t d_in, int64_t d_out, int64_t r, float gscale, void *stream);

/* [BLR] blr_backward_paths with one path. */
int blr_backward(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                 const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg, int64_t M, int64_t d_in,
                 int64_t d_out, int64_t r, float gscale, void *stream);

/* Bytes of device workspace blr_backward_ws / blr_backward_paths_ws need (0 on bad sizes). */
size_t blr_backward_workspace_size(int64_t M, int64_t d_in, int64_t d_out, int64_t r);

/* The backward with a caller-owned workspace of at least
 * blr_backward_workspace_size(...) bytes, 256-byte aligned, not overlapping the
 * outputs; calls sharing a workspace must not overlap in time. */
int blr_backward_paths_ws(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                          const float *g, const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg,
                          int64_t M, int64_t d_in, int64_t d_out, int64_t r, float gscale, void *workspace,
                          size_t workspace_bytes, void *stream);
int blr_backward_ws(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                    const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg, int64_t M,
                    int64_t d_in, int64_t d_out, int64_t r, float gscale, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Bytes of the buffer that keeps a layer's activations for its backward: per
 * path, a [M][r] then c [M][d_out], f32, each part 256-byte aligned (0 on bad
 * sizes). */
size_t blr_saved_size(int64_t P, int64_t M, int64_t d_in, int64_t d_out, int64_t r);

/* [BLR] blr_forward_paths that also keeps, per path, a = (x.g) S_V and
 * c = (a.l) S_U^T (the f32 values the forward computed) in `saved`, as the
 * page's blr_forward keeps a and c in its scratch for blr_backward.  y has the
 * bits blr_forward_paths gives.  saved: caller-owned device memory of at least
 * blr_saved_size(P, M, d_in, d_out, r) bytes, 256-byte aligned, overlapping
 * neither y nor the inputs; its previous contents are overwritten.  Otherwise as
 * blr_forward_paths (library-owned workspace).  Asynchronous on `stream`. */
int blr_forward_paths_save(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                           const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out,
                           int64_t r, void *saved, size_t saved_bytes, void *stream);

/* [BLR] blr_backward_paths from the activations a blr_forward_paths_save call
 * kept in `saved` (same P, M, d_in, d_out, r, bitmaps, h, l, g and x; this is
 * not checked): the page's blr_backward, which reads a and c from the forward
 * instead of recomputing them.  Per path, one pass over dy and c forms the sums
 * of dy.c and f16(dy.h.gscale), then db, dx' and the sums as in
 * blr_backward_paths: four launches per path instead of five, and the same bits
 * as blr_backward_paths.  saved must not overlap the outputs; everything else
 * as for blr_backward_paths.  Asynchronous on `stream`. */
int blr_backward_paths_saved(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h,
                             const float *l, const float *g, const float *x, const float *dy, float *dx, float *dh,
                             float *dl, float *dg, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float gscale,
                             const void *saved, size_t saved_bytes, void *stream);

/* Number of device allocations the library has made for its own workspaces
 * since the process started (grow-only: a call that fits the buffer its
 * (device, stream) already holds allocates nothing).  The page's GEMM keeps a
 * pooled buffer set whose allocation count stays constant once warmed up; this
 * counter lets a caller check the same.  tq2_gemm and tq2_dequant never
 * allocate. */
uint64_t tq2_workspace_allocs(void);

/* Static text for a status code. */
const char *tq2_strerror(int status);

/* Library version string. */
const char *tq2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBTQ2_H */
