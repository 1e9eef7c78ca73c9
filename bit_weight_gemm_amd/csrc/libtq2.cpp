// C ABI of libtq2: argument checks, host repack of the weight blocks, path choice
// and kernel launch.  Declarations and the contract live in include/libtq2.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <initializer_list>
#include <utility>
#include <new>
#include <vector>

#include "../../include/libtq2.h"
#include "internal.h"
#include "repack.h"

using tq2::DevWeight;

// Scratch of blr_forward_noalloc: a fixed device array of the library, one copy
// per GPU, held from module load until the process ends.  Host code never uses
// this name as an address: each device's copy is found once with
// hipGetSymbolAddress (scratch_address below) and that pointer is what kernels
// receive.
static __device__ __align__(256) unsigned char scratch[TQ2_STATIC_SCRATCH_BYTES];

struct tq2_weight {
    DevWeight dev;
    int device = -1;
};

namespace {

// gfx950 check, cached per device ordinal.
int check_device(int *dev_out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TQ2_ENODEV;
    static std::mutex mu;
    static std::vector<int> state;  // 0 unknown, 1 ok, -1 not gfx950
    std::lock_guard<std::mutex> lock(mu);
    if ((int)state.size() <= dev) state.resize(dev + 1, 0);
    if (state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TQ2_ENODEV;
        state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    }
    if (state[dev] != 1) return TQ2_ENODEV;
    if (dev_out) *dev_out = dev;
    return TQ2_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

int from_hip(hipError_t e) {
    if (e == hipSuccess) return TQ2_OK;
    if (e == hipErrorOutOfMemory) return TQ2_ENOMEM;
    return TQ2_EDEVICE;
}

std::atomic<int64_t> g_m_small{-1};
std::atomic<int> g_forced{-1};  // -1 unread, 0 none, 1 f32, 2 mfma

int64_t m_small() {
    int64_t v = g_m_small.load();
    if (v >= 0) return v;
    const char *s = std::getenv("TQ2_M_SMALL");
    v = (s && *s) ? std::strtoll(s, nullptr, 10) : 4;
    if (v < 0) v = 0;
    int64_t expect = -1;
    g_m_small.compare_exchange_strong(expect, v);
    return g_m_small.load();
}

int forced_path() {
    int v = g_forced.load();
    if (v >= 0) return v;
    const char *s = std::getenv("TQ2_PATH");
    v = 0;
    if (s && std::strcmp(s, "f32") == 0) v = TQ2_PATH_F32;
    if (s && std::strcmp(s, "mfma") == 0) v = TQ2_PATH_MFMA;
    g_forced.store(v);
    return v;
}


// Library-owned workspaces: one grow-only device buffer per (device, stream),
// kept until the process ends.  Calls on one stream are ordered by the stream,
// so they can share its buffer; a host-side lock is held from the size check
// until the launches are queued, so two host threads on one stream cannot free
// a buffer the other is about to use.
struct Pool {
    int dev = -1;
    hipStream_t stream = nullptr;
    void *ptr = nullptr;
    size_t bytes = 0;
    std::mutex mu;
};
std::mutex g_pools_mu;
std::vector<std::unique_ptr<Pool>> g_pools;
std::atomic<uint64_t> g_ws_allocs{0};  // device allocations made for workspaces

Pool &pool_for(int dev, hipStream_t s) {
    std::lock_guard<std::mutex> lock(g_pools_mu);
    for (auto &p : g_pools)
        if (p->dev == dev && p->stream == s) return *p;
    g_pools.emplace_back(new Pool);
    g_pools.back()->dev = dev;
    g_pools.back()->stream = s;
    return *g_pools.back();
}

// At least `need` bytes in the pool (call with pool.mu held).  Growing frees the
// old buffer first; hipFree waits for the device, so the work queued earlier on
// the stream has finished with it.
int pool_reserve(Pool &p, size_t need) {
    if (p.bytes >= need) return TQ2_OK;
    if (p.ptr) {
        const hipError_t e = hipFree(p.ptr);
        p.ptr = nullptr;
        p.bytes = 0;
        if (e != hipSuccess) return from_hip(e);
    }
    void *m = nullptr;
    const hipError_t e = hipMalloc(&m, need);
    if (e != hipSuccess) return from_hip(e);
    p.ptr = m;
    p.bytes = need;
    g_ws_allocs.fetch_add(1);
    return TQ2_OK;
}

// Device address of `scratch` on device `dev`, which must be the current device:
// looked up with hipGetSymbolAddress on the first call made on that device and
// kept (each GPU holds its own copy of the array, at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

int scratch_address(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return TQ2_ENODEV;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return TQ2_EDEVICE;
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return TQ2_OK;
}

}  // namespace

extern "C" {

const char *tq2_strerror(int status) {
    switch (status) {
        case TQ2_OK: return "ok";
        case TQ2_EINVAL: return "invalid argument";
        case TQ2_ENOMEM: return "out of memory";
        case TQ2_EDEVICE: return "HIP call or kernel launch failed";
        case TQ2_ENODEV: return "no gfx950 HIP device current";
        case TQ2_ETOOBIG: return "the call needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

const char *tq2_version(void) { return "libtq2 0.1 (gfx950)"; }

int64_t tq2_set_m_small(int64_t v) {
    const int64_t old = m_small();
    g_m_small.store(v < 0 ? 0 : v);
    return old;
}

int tq2_set_path(int path) {
    if (path < TQ2_PATH_AUTO || path > TQ2_PATH_MFMA) return TQ2_EINVAL;
    const int old = forced_path();
    g_forced.store(path);
    return old;
}

int tq2_select_path(int64_t M) {
    const int f = forced_path();
    if (f) return f;
    return M <= m_small() ? TQ2_PATH_F32 : TQ2_PATH_MFMA;
}

int tq2_upload(const void *aos, size_t nbytes, int64_t N, int64_t K, void *stream, tq2_weight **out) {
    if (!aos || !out) return TQ2_EINVAL;
    if (N < 1 || K < tq2::kBlock || K % tq2::kBlock) return TQ2_EINVAL;
    const int64_t kb = K / tq2::kBlock;
    // kernels index rows with 32-bit integers: the padded row count must fit
    if (N > ((int64_t)1 << 31) - tq2::kRowPad || K > (int64_t)1 << 30) return TQ2_EINVAL;
    if (nbytes != (size_t)N * (size_t)kb * tq2::kBlockBytes) return TQ2_EINVAL;
    *out = nullptr;
    int dev = -1;
    int st = check_device(&dev);
    if (st) return st;

    const tq2::RepackLayout L = tq2::repack_layout(N, K);
    const size_t total = L.total;
    bool mfma_ok = true;
    std::vector<uint8_t> host;
    try {
        host.resize(total);
    } catch (const std::bad_alloc &) {
        return TQ2_ENOMEM;
    }
    if (!tq2::repack_blocks(static_cast<const uint8_t *>(aos), L, host.data(), &mfma_ok)) return TQ2_EINVAL;

    tq2_weight *w = new (std::nothrow) tq2_weight;
    if (!w) return TQ2_ENOMEM;
    void *dmem = nullptr;
    hipError_t e = hipMalloc(&dmem, total);
    if (e != hipSuccess) {
        delete w;
        return from_hip(e);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    e = hipMemcpyAsync(dmem, host.data(), total, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        (void)hipFree(dmem);
        delete w;
        return from_hip(e);
    }
    w->device = dev;
    w->dev.N = N;
    w->dev.K = K;
    w->dev.Npad = L.npad;
    w->dev.codes = static_cast<uint32_t *>(dmem);
    w->dev.scales = reinterpret_cast<uint16_t *>(static_cast<char *>(dmem) + L.scale_off);
    w->dev.bytes = total;
    w->dev.mfma_ok = mfma_ok;
    *out = w;
    return TQ2_OK;
}

int tq2_free(tq2_weight *w) {
    if (!w) return TQ2_OK;
    hipError_t e = hipSuccess;
    if (w->dev.codes) e = hipFree(w->dev.codes);
    delete w;
    return from_hip(e);
}

int tq2_weight_info(const tq2_weight *w, int64_t *N, int64_t *K, size_t *device_bytes) {
    if (!w) return TQ2_EINVAL;
    if (N) *N = w->dev.N;
    if (K) *K = w->dev.K;
    if (device_bytes) *device_bytes = w->dev.bytes;
    return TQ2_OK;
}

static int check_weight_call(const tq2_weight *w, int64_t N, int64_t K, int *dev) {
    if (!w || N != w->dev.N || K != w->dev.K) return TQ2_EINVAL;
    int st = check_device(dev);
    if (st) return st;
    if (*dev != w->device) return TQ2_EINVAL;  // handle lives on another device
    return TQ2_OK;
}

int tq2_gemm_path(const tq2_weight *w, const float *x, float *y, int64_t M, int64_t N, int64_t K, int path,
                  void *stream) {
    if (M < 0 || path < TQ2_PATH_AUTO || path > TQ2_PATH_MFMA) return TQ2_EINVAL;
    if (M > ((int64_t)1 << 31) - 1) return TQ2_EINVAL;
    int dev = -1;
    int st = check_weight_call(w, N, K, &dev);
    if (st) return st;
    if (M == 0) return TQ2_OK;
    if (!x || !y || !aligned16(x) || !aligned16(y)) return TQ2_EINVAL;
    if (overlap(x, (size_t)M * K * 4, y, (size_t)M * N * 4)) return TQ2_EINVAL;
    if (path == TQ2_PATH_AUTO) path = tq2_select_path(M);
    if (path == TQ2_PATH_MFMA && !w->dev.mfma_ok) path = TQ2_PATH_F32;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (path == TQ2_PATH_F32)
        e = tq2::launch_gemv_f32(w->dev, x, y, M, s);
    else if (tq2::skinny_fits(w->dev, M))
        e = tq2::launch_skinny(w->dev, x, y, M, dev, s);
    else
        e = tq2::launch_gemm_mfma(w->dev, x, y, M, s);
    return from_hip(e);
}

int tq2_gemm(const tq2_weight *w, const float *x, float *y, int64_t M, int64_t N, int64_t K, void *stream) {
    return tq2_gemm_path(w, x, y, M, N, K, TQ2_PATH_AUTO, stream);
}

int tq2_dequant(const tq2_weight *w, float *w_out, void *stream) {
    int dev = -1;
    if (!w) return TQ2_EINVAL;
    int st = check_weight_call(w, w->dev.N, w->dev.K, &dev);
    if (st) return st;
    if (!w_out || !aligned16(w_out)) return TQ2_EINVAL;
    return from_hip(tq2::launch_dequant(w->dev, w_out, static_cast<hipStream_t>(stream)));
}

size_t blr_workspace_size(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    if (M < 0 || d_in < 1 || d_out < 1 || r < 32 || r % 32) return 0;
    if (M > ((int64_t)1 << 31) - 1 || d_in > ((int64_t)1 << 30) || d_out > ((int64_t)1 << 30) ||
        r > ((int64_t)1 << 30))
        return 0;
    const size_t total = tq2::blr_plan(M, d_in, d_out, r).total;
    return total > 256 ? total : 256;  // 0 means bad sizes: valid ones get at least one 256-byte unit
}

size_t blr_backward_workspace_size(int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    if (blr_workspace_size(M, d_in, d_out, r) == 0) return 0;
    return tq2::blr_bwd_plan(M, d_in, d_out, r).total;
}

uint64_t tq2_workspace_allocs(void) { return g_ws_allocs.load(); }

}  // extern "C"

namespace {

// The kernels read each path's sign bitmaps with 32-bit byte offsets: each, with
// the 512 rows of padding its products may step past its end, under 2 GB.
bool bitmaps_fit(int64_t d_in, int64_t d_out, int64_t r) {
    const int64_t lim = (int64_t)1 << 31;
    return (d_in + 512) * (r / 32) * 4 < lim && (d_out + 512) * (r / 32) * 4 < lim;
}

// Host-side checks of a BLR forward: P stacked paths of the given sizes, every
// pointer and alignment, and y overlapping none of the inputs.  The workspace is
// checked by the caller (it may be the library's own).
int blr_forward_check(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                      const float *g, const float *x, const float *y, int64_t M, int64_t d_in, int64_t d_out,
                      int64_t r) {
    if (blr_workspace_size(M, d_in, d_out, r) == 0 || P < 1 || P > 4096 || !bitmaps_fit(d_in, d_out, r))
        return TQ2_EINVAL;
    if (M == 0) return TQ2_OK;
    if (!bits_u || !bits_v || !h || !l || !g || !x || !y) return TQ2_EINVAL;
    if (!aligned16(y) || (reinterpret_cast<uintptr_t>(x) & 3u) || (reinterpret_cast<uintptr_t>(bits_u) & 3u) ||
        (reinterpret_cast<uintptr_t>(bits_v) & 3u) || (reinterpret_cast<uintptr_t>(h) & 3u) ||
        (reinterpret_cast<uintptr_t>(l) & 3u) || (reinterpret_cast<uintptr_t>(g) & 3u))
        return TQ2_EINVAL;
    const size_t ybytes = (size_t)M * d_out * 4, p = (size_t)P;
    if (overlap(y, ybytes, x, (size_t)M * d_in * 4) || overlap(y, ybytes, bits_u, p * d_out * (r / 32) * 4) ||
        overlap(y, ybytes, bits_v, p * d_in * (r / 32) * 4) || overlap(y, ybytes, h, p * d_out * 4) ||
        overlap(y, ybytes, l, p * r * 4) || overlap(y, ybytes, g, p * d_in * 4))
        return TQ2_EINVAL;
    return TQ2_OK;
}

// The caller's workspace: large enough, 256-byte aligned, not overlapping the output.
int workspace_check(const void *ws, size_t ws_bytes, size_t need, const void *out, size_t out_bytes) {
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return TQ2_EINVAL;
    if (overlap(out, out_bytes, ws, need)) return TQ2_EINVAL;
    return TQ2_OK;
}

// Saved activations of a layer's forward (blr_forward_paths_save): per path, a
// [M][r] then c [M][d_out], f32, each 256-byte aligned.
struct SavedLayout {
    size_t a_bytes, c_off, path_bytes;
};
SavedLayout saved_layout(int64_t M, int64_t d_out, int64_t r) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    SavedLayout L{};
    L.a_bytes = up((size_t)M * r * 4);
    L.c_off = L.a_bytes;
    L.path_bytes = L.c_off + up((size_t)M * d_out * 4);
    return L;
}

// The paths one after another, sharing one path's workspace (checked arguments);
// with `saved`, each path also keeps its a and c there.
int blr_forward_launch(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                       const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                       void *workspace, hipStream_t s, void *saved = nullptr) {
    const tq2::BlrPlan plan = tq2::blr_plan(M, d_in, d_out, r);
    const SavedLayout sl = saved_layout(M, d_out, r);
    const int64_t wu = d_out * (r / 32), wv = d_in * (r / 32);
    for (int64_t p = 0; p < P; ++p) {
        char *sp = saved ? static_cast<char *>(saved) + (size_t)p * sl.path_bytes : nullptr;
        float *sa = sp ? reinterpret_cast<float *>(sp) : nullptr;
        float *sc = sp ? reinterpret_cast<float *>(sp + sl.c_off) : nullptr;
        const int st = from_hip(tq2::launch_blr_forward(plan, bits_u + p * wu, bits_v + p * wv, h + p * d_out,
                                                        l + p * r, g + p * d_in, x, y, workspace, p > 0, sa, sc, s));
        if (st) return st;
    }
    return TQ2_OK;
}

// Host-side checks of a BLR backward (everything but the workspace).
int blr_backward_check(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                       const float *g, const float *x, const float *dy, const float *dx, const float *dh,
                       const float *dl, const float *dg, int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                       float gscale) {
    if (blr_backward_workspace_size(M, d_in, d_out, r) == 0 || P < 1 || P > 4096 || !bitmaps_fit(d_in, d_out, r))
        return TQ2_EINVAL;
    int e2 = 0;
    if (!std::isfinite(gscale) || gscale <= 0.0f || std::frexp(gscale, &e2) != 0.5f || gscale > 65536.0f)
        return TQ2_EINVAL;  // a power of two, at most 2^16
    if (!bits_u || !bits_v || !h || !l || !g || !x || !dy || !dx || !dh || !dl || !dg) return TQ2_EINVAL;
    const uintptr_t mis = reinterpret_cast<uintptr_t>(bits_u) | reinterpret_cast<uintptr_t>(bits_v) |
                          reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(g) |
                          reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(dy) |
                          reinterpret_cast<uintptr_t>(dx) | reinterpret_cast<uintptr_t>(dh) |
                          reinterpret_cast<uintptr_t>(dl) | reinterpret_cast<uintptr_t>(dg);
    if ((mis & 3u) || (reinterpret_cast<uintptr_t>(l) & 15u)) return TQ2_EINVAL;
    const size_t p = (size_t)P;
    struct Span { const void *ptr; size_t bytes; };
    const Span outs[] = {{dx, (size_t)M * d_in * 4}, {dh, p * d_out * 4}, {dl, p * r * 4}, {dg, p * d_in * 4}};
    const Span ins[] = {{bits_u, p * d_out * (r / 32) * 4}, {bits_v, p * d_in * (r / 32) * 4}, {h, p * d_out * 4},
                        {l, p * r * 4}, {g, p * d_in * 4}, {x, (size_t)M * d_in * 4}, {dy, (size_t)M * d_out * 4}};
    for (size_t i = 0; i < 4; ++i) {
        for (const Span &in : ins)
            if (outs[i].bytes && in.bytes && overlap(outs[i].ptr, outs[i].bytes, in.ptr, in.bytes)) return TQ2_EINVAL;
        for (size_t j = i + 1; j < 4; ++j)
            if (outs[i].bytes && outs[j].bytes && overlap(outs[i].ptr, outs[i].bytes, outs[j].ptr, outs[j].bytes))
                return TQ2_EINVAL;
    }
    return TQ2_OK;
}

// The caller's backward workspace must also stay clear of all four outputs.
int backward_workspace_check(const void *ws, size_t ws_bytes, size_t need, int64_t P, const float *dx,
                             const float *dh, const float *dl, const float *dg, int64_t M, int64_t d_in,
                             int64_t d_out, int64_t r) {
    const size_t p = (size_t)P;
    int st = workspace_check(ws, ws_bytes, need, dx, (size_t)M * d_in * 4);
    if (!st) st = workspace_check(ws, ws_bytes, need, dh, p * d_out * 4);
    if (!st) st = workspace_check(ws, ws_bytes, need, dl, p * r * 4);
    if (!st) st = workspace_check(ws, ws_bytes, need, dg, p * d_in * 4);
    return st;
}

int blr_backward_launch(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                        const float *g, const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg,
                        int64_t M, int64_t d_in, int64_t d_out, int64_t r, float gscale, void *workspace,
                        hipStream_t s, const void *saved = nullptr) {
    const tq2::BlrBwdPlan plan = tq2::blr_bwd_plan(M, d_in, d_out, r);
    const SavedLayout sl = saved_layout(M, d_out, r);
    const int64_t wu = d_out * (r / 32), wv = d_in * (r / 32);
    for (int64_t q = 0; q < P; ++q) {
        hipError_t e;
        if (saved) {
            const char *sp = static_cast<const char *>(saved) + (size_t)q * sl.path_bytes;
            e = tq2::launch_blr_backward_saved(plan, bits_u + q * wu, bits_v + q * wv, h + q * d_out, l + q * r,
                                               g + q * d_in, x, dy, reinterpret_cast<const float *>(sp),
                                               reinterpret_cast<const float *>(sp + sl.c_off), dx, dh + q * d_out,
                                               dl + q * r, dg + q * d_in, gscale, workspace, q > 0, s);
        } else {
            e = tq2::launch_blr_backward(plan, bits_u + q * wu, bits_v + q * wv, h + q * d_out, l + q * r,
                                         g + q * d_in, x, dy, dx, dh + q * d_out, dl + q * r, dg + q * d_in, gscale,
                                         workspace, q > 0, s);
        }
        const int st = from_hip(e);
        if (st) return st;
    }
    return TQ2_OK;
}

// The caller's buffer of saved activations: large enough for P paths, 256-byte
// aligned, clear of the buffers listed (which it must not overlap).
int saved_check(const void *saved, size_t saved_bytes, int64_t P, int64_t M, int64_t d_out, int64_t r,
                std::initializer_list<std::pair<const void *, size_t>> others) {
    const size_t need = (size_t)P * saved_layout(M, d_out, r).path_bytes;
    if (!saved || saved_bytes < need || (reinterpret_cast<uintptr_t>(saved) & 255u)) return TQ2_EINVAL;
    for (const auto &o : others)
        if (overlap(saved, need, o.first, o.second)) return TQ2_EINVAL;
    return TQ2_OK;
}

}  // namespace

extern "C" {

int blr_forward_paths_ws(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                         const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                         void *workspace, size_t workspace_bytes, void *stream) {
    int st = blr_forward_check(P, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r);
    if (st) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st || M == 0) return st;
    st = workspace_check(workspace, workspace_bytes, blr_workspace_size(M, d_in, d_out, r), y, (size_t)M * d_out * 4);
    if (st) return st;
    return blr_forward_launch(P, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r, workspace,
                              static_cast<hipStream_t>(stream));
}

int blr_forward_ws(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                   const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out, int64_t r, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return blr_forward_paths_ws(1, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r, workspace, workspace_bytes,
                                stream);
}

int blr_forward_paths(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                      const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                      void *stream) {
    int st = blr_forward_check(P, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r);
    if (st) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st || M == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Pool &pool = pool_for(dev, s);
    std::lock_guard<std::mutex> lock(pool.mu);  // held until the launches are queued
    st = pool_reserve(pool, blr_workspace_size(M, d_in, d_out, r));
    if (st) return st;
    return blr_forward_launch(P, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r, pool.ptr, s);
}

int blr_forward(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out, int64_t r, void *stream) {
    return blr_forward_paths(1, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r, stream);
}

int blr_forward_noalloc(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                        const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out, int64_t r,
                        void *stream) {
    const size_t need = blr_workspace_size(M, d_in, d_out, r);
    if (need == 0 || !bitmaps_fit(d_in, d_out, r)) return TQ2_EINVAL;
    if (need > (size_t)TQ2_STATIC_SCRATCH_BYTES) return TQ2_ETOOBIG;  // sizes first: nothing else is looked at
    int st = blr_forward_check(1, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r);
    if (st) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st || M == 0) return st;
    void *ws = nullptr;
    st = scratch_address(dev, &ws);
    if (st) return st;
    // every byte of the workspace that the launches read, they first write: no clearing needed
    return blr_forward_launch(1, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r, ws,
                              static_cast<hipStream_t>(stream));
}

size_t blr_saved_size(int64_t P, int64_t M, int64_t d_in, int64_t d_out, int64_t r) {
    if (P < 1 || P > 4096 || blr_workspace_size(M, d_in, d_out, r) == 0) return 0;
    const size_t total = (size_t)P * saved_layout(M, d_out, r).path_bytes;
    return total > 256 ? total : 256;  // 0 means bad sizes
}

int blr_forward_paths_save(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                           const float *g, const float *x, float *y, int64_t M, int64_t d_in, int64_t d_out,
                           int64_t r, void *saved, size_t saved_bytes, void *stream) {
    int st = blr_forward_check(P, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r);
    if (st) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st || M == 0) return st;
    const size_t p = (size_t)P;
    st = saved_check(saved, saved_bytes, P, M, d_out, r,
                     {{y, (size_t)M * d_out * 4}, {x, (size_t)M * d_in * 4}, {bits_u, p * d_out * (r / 32) * 4},
                      {bits_v, p * d_in * (r / 32) * 4}, {h, p * d_out * 4}, {l, p * r * 4}, {g, p * d_in * 4}});
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Pool &pool = pool_for(dev, s);
    std::lock_guard<std::mutex> lock(pool.mu);
    st = pool_reserve(pool, blr_workspace_size(M, d_in, d_out, r));
    if (st) return st;
    return blr_forward_launch(P, bits_u, bits_v, h, l, g, x, y, M, d_in, d_out, r, pool.ptr, s, saved);
}

int blr_backward_paths_saved(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h,
                             const float *l, const float *g, const float *x, const float *dy, float *dx, float *dh,
                             float *dl, float *dg, int64_t M, int64_t d_in, int64_t d_out, int64_t r, float gscale,
                             const void *saved, size_t saved_bytes, void *stream) {
    int st = blr_backward_check(P, bits_u, bits_v, h, l, g, x, dy, dx, dh, dl, dg, M, d_in, d_out, r, gscale);
    if (st) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st || M == 0) return st;
    const size_t p = (size_t)P;
    st = saved_check(saved, saved_bytes, P, M, d_out, r,
                     {{dx, (size_t)M * d_in * 4}, {dh, p * d_out * 4}, {dl, p * r * 4}, {dg, p * d_in * 4}});
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Pool &pool = pool_for(dev, s);
    std::lock_guard<std::mutex> lock(pool.mu);
    st = pool_reserve(pool, blr_backward_workspace_size(M, d_in, d_out, r));
    if (st) return st;
    return blr_backward_launch(P, bits_u, bits_v, h, l, g, x, dy, dx, dh, dl, dg, M, d_in, d_out, r, gscale, pool.ptr,
                               s, saved);
}

int blr_backward_paths_ws(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                          const float *g, const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg,
                          int64_t M, int64_t d_in, int64_t d_out, int64_t r, float gscale, void *workspace,
                          size_t workspace_bytes, void *stream) {
    int st = blr_backward_check(P, bits_u, bits_v, h, l, g, x, dy, dx, dh, dl, dg, M, d_in, d_out, r, gscale);
    if (st) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st) return st;
    const size_t need = blr_backward_workspace_size(M, d_in, d_out, r);
    st = backward_workspace_check(workspace, workspace_bytes, need, P, dx, dh, dl, dg, M, d_in, d_out, r);
    if (st || M == 0) return st;  // no tokens: no gradient to add, dx is empty
    return blr_backward_launch(P, bits_u, bits_v, h, l, g, x, dy, dx, dh, dl, dg, M, d_in, d_out, r, gscale,
                               workspace, static_cast<hipStream_t>(stream));
}

int blr_backward_ws(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                    const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg, int64_t M,
                    int64_t d_in, int64_t d_out, int64_t r, float gscale, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return blr_backward_paths_ws(1, bits_u, bits_v, h, l, g, x, dy, dx, dh, dl, dg, M, d_in, d_out, r, gscale,
                                 workspace, workspace_bytes, stream);
}

int blr_backward_paths(int64_t P, const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l,
                       const float *g, const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg,
                       int64_t M, int64_t d_in, int64_t d_out, int64_t r, float gscale, void *stream) {
    int st = blr_backward_check(P, bits_u, bits_v, h, l, g, x, dy, dx, dh, dl, dg, M, d_in, d_out, r, gscale);
    if (st) return st;
    int dev = -1;
    st = check_device(&dev);
    if (st || M == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Pool &pool = pool_for(dev, s);
    std::lock_guard<std::mutex> lock(pool.mu);
    st = pool_reserve(pool, blr_backward_workspace_size(M, d_in, d_out, r));
    if (st) return st;
    return blr_backward_launch(P, bits_u, bits_v, h, l, g, x, dy, dx, dh, dl, dg, M, d_in, d_out, r, gscale, pool.ptr,
                               s);
}

int blr_backward(const uint32_t *bits_u, const uint32_t *bits_v, const float *h, const float *l, const float *g,
                 const float *x, const float *dy, float *dx, float *dh, float *dl, float *dg, int64_t M, int64_t d_in,
                 int64_t d_out, int64_t r, float gscale, void *stream) {
    return blr_backward_paths(1, bits_u, bits_v, h, l, g, x, dy, dx, dh, dl, dg, M, d_in, d_out, r, gscale, stream);
}

}  // extern "C"
