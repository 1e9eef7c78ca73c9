"""Python binding of libtq2 (ctypes): argument marshalling only.

Every step of the computation runs in the HIP kernels of libtq2.so; torch only
supplies device memory (tensors on the current GPU) and the current stream.
There is no CPU fallback: if the library is missing or fails to load, the calls
raise.

Names follow the C ABI in include/libtq2.h: tq2_upload, tq2_free, tq2_gemm,
tq2_gemm_path, tq2_dequant, blr_forward, blr_forward_paths, blr_backward_paths
(library-owned workspace), blr_forward_ws, blr_forward_paths_ws,
blr_backward_paths_ws (caller-owned workspace), blr_forward_paths_save and
blr_backward_paths_saved (activations kept by the forward for the backward),
blr_saved_size, blr_workspace_size,
blr_backward_workspace_size, tq2_workspace_allocs, tq2_select_path,
tq2_set_path, tq2_set_m_small, tq2_strerror, tq2_version.

Every tensor's shape is checked here against the sizes the call derives from x,
h and l before anything reaches the library: the C ABI takes raw device
pointers and cannot see buffer sizes.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq2.so")

TQ2_OK, TQ2_EINVAL, TQ2_ENOMEM, TQ2_EDEVICE, TQ2_ENODEV, TQ2_ETOOBIG = 0, -1, -2, -3, -4, -5
TQ2_STATIC_SCRATCH_BYTES = 16 << 20
TQ2_PATH_AUTO, TQ2_PATH_F32, TQ2_PATH_MFMA = 0, 1, 2

_lib = None


class Tq2Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {tq2_strerror(status)} ({status})")


def _single_hip_runtime():
    """Fail if two different HIP runtimes are mapped (device pointers would not mix)."""
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(f"more than one HIP runtime loaded: {sorted(real)}")


def lib():
    """Load libtq2.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- load torch's HIP runtime first

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run bit_weight_gemm_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    _single_hip_runtime()
    i64, sz, p, i32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    sig = {
        "tq2_upload": ([p, sz, i64, i64, p, ctypes.POINTER(p)], i32),
        "tq2_free": ([p], i32),
        "tq2_weight_info": ([p, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(sz)], i32),
        "tq2_gemm": ([p, p, p, i64, i64, i64, p], i32),
        "tq2_gemm_path": ([p, p, p, i64, i64, i64, i32, p], i32),
        "tq2_select_path": ([i64], i32),
        "tq2_set_m_small": ([i64], i64),
        "tq2_dequant": ([p, p, p], i32),
        "tq2_set_path": ([i32], i32),
        "tq2_workspace_allocs": ([], ctypes.c_uint64),
        "blr_workspace_size": ([i64, i64, i64, i64], sz),
        "blr_forward": ([p, p, p, p, p, p, p, i64, i64, i64, i64, p], i32),
        "blr_forward_paths": ([i64, p, p, p, p, p, p, p, i64, i64, i64, i64, p], i32),
        "blr_forward_noalloc": ([p, p, p, p, p, p, p, i64, i64, i64, i64, p], i32),
        "blr_forward_ws": ([p, p, p, p, p, p, p, i64, i64, i64, i64, p, sz, p], i32),
        "blr_forward_paths_ws": ([i64, p, p, p, p, p, p, p, i64, i64, i64, i64, p, sz, p], i32),
        "blr_backward_workspace_size": ([i64, i64, i64, i64], sz),
        "blr_backward_paths": ([i64, p, p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_float, p], i32),
        "blr_backward": ([p, p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_float, p], i32),
        "blr_backward_paths_ws": ([i64, p, p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_float, p, sz,
                                   p], i32),
        "blr_backward_ws": ([p, p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_float, p, sz, p], i32),
        "blr_saved_size": ([i64, i64, i64, i64, i64], sz),
        "blr_forward_paths_save": ([i64, p, p, p, p, p, p, p, i64, i64, i64, i64, p, sz, p], i32),
        "blr_backward_paths_saved": ([i64, p, p, p, p, p, p, p, p, p, p, p, i64, i64, i64, i64, ctypes.c_float, p, sz,
                                      p], i32),
        "tq2_strerror": ([i32], ctypes.c_char_p),
        "tq2_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(status: int, what: str):
    if status != TQ2_OK:
        raise Tq2Error(status, what)


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, dtype, name):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def tq2_strerror(status: int) -> str:
    return lib().tq2_strerror(int(status)).decode()


def tq2_version() -> str:
    return lib().tq2_version().decode()


def tq2_select_path(m: int) -> int:
    return int(lib().tq2_select_path(int(m)))


def tq2_set_m_small(v: int) -> int:
    return int(lib().tq2_set_m_small(int(v)))


def tq2_set_path(path: int) -> int:
    """Force the path of every auto call (TQ2_PATH_AUTO restores the choice by M); returns the old setting."""
    st = int(lib().tq2_set_path(int(path)))
    if st < 0:
        raise Tq2Error(st, "tq2_set_path")
    return st


def tq2_workspace_allocs() -> int:
    """Device allocations the library has made for its own (grow-only) workspaces."""
    return int(lib().tq2_workspace_allocs())


def blr_workspace_size(m: int, d_in: int, d_out: int, r: int) -> int:
    return int(lib().blr_workspace_size(int(m), int(d_in), int(d_out), int(r)))


class Tq2Weight:
    """Device handle of an uploaded TQ2_0_g128 weight [N][K]; freed on close()/GC."""

    def __init__(self, handle: ctypes.c_void_p, n: int, k: int):
        self._h = handle
        self.N, self.K = n, k

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("weight already freed")
        return self._h

    def device_bytes(self) -> int:
        nb = ctypes.c_size_t()
        _check(lib().tq2_weight_info(self.handle, None, None, ctypes.byref(nb)), "tq2_weight_info")
        return nb.value

    def close(self):
        if self._h is not None:
            h, self._h = self._h, None
            _check(lib().tq2_free(h), "tq2_free")

    def __del__(self):
        try:
            if self._h is not None and _lib is not None:
                _lib.tq2_free(self._h)
                self._h = None
        except Exception:
            pass


def tq2_upload(aos, n: int, k: int, stream=None) -> Tq2Weight:
    """Upload AoS block bytes (numpy uint8 / bytes) for a weight [n][k]."""
    buf = np.ascontiguousarray(np.frombuffer(aos, np.uint8) if isinstance(aos, (bytes, bytearray)) else aos,
                               dtype=np.uint8)
    out = ctypes.c_void_p()
    _check(lib().tq2_upload(buf.ctypes.data_as(ctypes.c_void_p), buf.size, int(n), int(k), _stream(stream),
                            ctypes.byref(out)), "tq2_upload")
    return Tq2Weight(out, int(n), int(k))


def tq2_free(w: Tq2Weight):
    w.close()


def tq2_gemm_path(w: Tq2Weight, x, y=None, path: int = TQ2_PATH_AUTO, stream=None):
    """y[M][N] = x[M][K] @ W^T on the chosen path; returns y (allocated if None)."""
    import torch

    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError(f"x must be [M, {w.K}]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, w.N), dtype=torch.float32, device=x.device)
    if y.shape != (m, w.N):
        raise ValueError(f"y must be [{m}, {w.N}]")
    _check(lib().tq2_gemm_path(w.handle, _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"), m, w.N, w.K,
                               int(path), _stream(stream)), "tq2_gemm")
    return y


def tq2_gemm(w: Tq2Weight, x, y=None, stream=None):
    return tq2_gemm_path(w, x, y, TQ2_PATH_AUTO, stream)


def tq2_dequant(w: Tq2Weight, out=None, stream=None):
    import torch

    if out is None:
        out = torch.empty((w.N, w.K), dtype=torch.float32, device="cuda")
    if tuple(out.shape) != (w.N, w.K):
        raise ValueError(f"out must be [{w.N}, {w.K}]")
    _check(lib().tq2_dequant(w.handle, _dev(out, torch.float32, "out"), _stream(stream)), "tq2_dequant")
    return out


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _blr_sizes(bits_u, bits_v, h, l, g, x, paths: bool):
    """(P, M, d_in, d_out, r) from x, h and l, with every operand's shape checked
    against them (bits as int32 words: [P][d_out][r/32] and [P][d_in][r/32])."""
    if x.dim() != 2:
        raise ValueError("x must be [M, d_in]")
    m, d_in = x.shape
    if paths:
        if h.dim() != 2 or l.dim() != 2:
            raise ValueError("h and l must be [P, d_out] and [P, r]")
        npaths, d_out = h.shape
        r = l.shape[1]
        lead = (npaths,)
    else:
        if h.dim() != 1 or l.dim() != 1:
            raise ValueError("h and l must be [d_out] and [r]")
        npaths, d_out, r = 1, h.shape[0], l.shape[0]
        lead = ()
    if r % 32:
        raise ValueError(f"r must be a multiple of 32, got {r}")
    _shape(l, lead + (r,), "l")
    _shape(g, lead + (d_in,), "g")
    _shape(bits_u, lead + (d_out, r // 32), "bits_u")
    _shape(bits_v, lead + (d_in, r // 32), "bits_v")
    return npaths, m, d_in, d_out, r


def _workspace(workspace, need, like, stream, what):
    """A caller workspace checked for size, or a temporary one tied to `stream`."""
    import torch

    if need == 0:
        raise Tq2Error(TQ2_EINVAL, what)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=like.device)
        if stream is not None and hasattr(stream, "cuda_stream"):
            workspace.record_stream(stream)  # not reused before the work queued on `stream` is done
    if workspace.numel() < need:
        raise ValueError(f"workspace needs {need} bytes, got {workspace.numel()}")
    return workspace


def _blr_forward_call(bits_u, bits_v, h, l, g, x, y, stream, paths: bool, workspace=None, use_ws=False):
    import torch

    npaths, m, d_in, d_out, r = _blr_sizes(bits_u, bits_v, h, l, g, x, paths)
    if y is None:
        y = torch.empty((m, d_out), dtype=torch.float32, device=x.device)
    _shape(y, (m, d_out), "y")
    args = [_dev(bits_u, torch.int32, "bits_u"), _dev(bits_v, torch.int32, "bits_v"), _dev(h, torch.float32, "h"),
            _dev(l, torch.float32, "l"), _dev(g, torch.float32, "g"), _dev(x, torch.float32, "x"),
            _dev(y, torch.float32, "y"), m, d_in, d_out, r]
    if use_ws:
        ws = _workspace(workspace, blr_workspace_size(m, d_in, d_out, r), x, stream, "blr_workspace_size")
        args += [_dev(ws, torch.uint8, "workspace"), ws.numel()]
    args.append(_stream(stream))
    L = lib()
    if paths:
        fn = L.blr_forward_paths_ws if use_ws else L.blr_forward_paths
        _check(fn(npaths, *args), fn.__name__)
    else:
        fn = L.blr_forward_ws if use_ws else L.blr_forward
        _check(fn(*args), fn.__name__)
    return y


def blr_forward(bits_u, bits_v, h, l, g, x, y=None, stream=None):
    """Binary low-rank layer forward (library-owned workspace); bits_* are int32
    tensors holding the u32 bitmap words [d_out][r/32] and [d_in][r/32]."""
    return _blr_forward_call(bits_u, bits_v, h, l, g, x, y, stream, paths=False)


def blr_forward_ws(bits_u, bits_v, h, l, g, x, y=None, workspace=None, stream=None):
    """blr_forward with a caller-owned workspace (uint8, >= blr_workspace_size bytes)."""
    return _blr_forward_call(bits_u, bits_v, h, l, g, x, y, stream, paths=False, workspace=workspace, use_ws=True)


def blr_forward_paths(bits_u, bits_v, h, l, g, x, y=None, stream=None):
    """A layer of P paths, y = sum_p h_p . c_p, rounded path by path; the per-path
    operands are stacked along a leading P axis (bits_u [P][d_out][r/32], bits_v
    [P][d_in][r/32], h [P][d_out], l [P][r], g [P][d_in])."""
    return _blr_forward_call(bits_u, bits_v, h, l, g, x, y, stream, paths=True)


def blr_forward_paths_ws(bits_u, bits_v, h, l, g, x, y=None, workspace=None, stream=None):
    return _blr_forward_call(bits_u, bits_v, h, l, g, x, y, stream, paths=True, workspace=workspace, use_ws=True)


def blr_backward_workspace_size(m: int, d_in: int, d_out: int, r: int) -> int:
    return int(lib().blr_backward_workspace_size(m, d_in, d_out, r))


def blr_saved_size(paths: int, m: int, d_in: int, d_out: int, r: int) -> int:
    return int(lib().blr_saved_size(int(paths), int(m), int(d_in), int(d_out), int(r)))


def blr_forward_paths_save(bits_u, bits_v, h, l, g, x, y=None, saved=None, stream=None):
    """blr_forward_paths that also keeps each path's a and c (f32) in `saved` (uint8,
    >= blr_saved_size bytes; allocated if None) for blr_backward_paths_saved.
    Returns (y, saved)."""
    import torch

    npaths, m, d_in, d_out, r = _blr_sizes(bits_u, bits_v, h, l, g, x, paths=True)
    if y is None:
        y = torch.empty((m, d_out), dtype=torch.float32, device=x.device)
    _shape(y, (m, d_out), "y")
    need = blr_saved_size(npaths, m, d_in, d_out, r)
    if need == 0:
        raise Tq2Error(TQ2_EINVAL, "blr_saved_size")
    if saved is None:
        saved = torch.empty(need, dtype=torch.uint8, device=x.device)
    if saved.dim() != 1 or saved.numel() < need:
        raise ValueError(f"saved must be a flat uint8 tensor of at least {need} bytes")
    _check(lib().blr_forward_paths_save(
        npaths, _dev(bits_u, torch.int32, "bits_u"), _dev(bits_v, torch.int32, "bits_v"),
        _dev(h, torch.float32, "h"), _dev(l, torch.float32, "l"), _dev(g, torch.float32, "g"),
        _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"), m, d_in, d_out, r,
        _dev(saved, torch.uint8, "saved"), saved.numel(), _stream(stream)), "blr_forward_paths_save")
    return y, saved


def blr_saved_views(saved, paths: int, m: int, d_out: int, r: int):
    """Per-path views (a [M][r], c [M][d_out]) of a buffer filled by blr_forward_paths_save."""
    import torch

    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    a_bytes = up(m * r * 4)
    path_bytes = a_bytes + up(m * d_out * 4)
    out = []
    for q in range(paths):
        base = q * path_bytes
        a = saved[base: base + m * r * 4].view(torch.float32).view(m, r)
        c = saved[base + a_bytes: base + a_bytes + m * d_out * 4].view(torch.float32).view(m, d_out)
        out.append((a, c))
    return out


def blr_backward_paths_saved(bits_u, bits_v, h, l, g, x, dy, dh, dl, dg, saved, dx=None, gscale=1024.0,
                             stream=None):
    """blr_backward_paths from the activations blr_forward_paths_save kept in `saved`
    (same layer and x): no recomputation, the same bits."""
    return _blr_backward_call(bits_u, bits_v, h, l, g, x, dy, dh, dl, dg, dx, gscale, stream, None, False,
                              saved=saved)


def _blr_backward_call(bits_u, bits_v, h, l, g, x, dy, dh, dl, dg, dx, gscale, stream, workspace, use_ws,
                       saved=None):
    import torch

    npaths, m, d_in, d_out, r = _blr_sizes(bits_u, bits_v, h, l, g, x, paths=True)
    _shape(dy, (m, d_out), "dy")
    _shape(dh, (npaths, d_out), "dh")
    _shape(dl, (npaths, r), "dl")
    _shape(dg, (npaths, d_in), "dg")
    if dx is None:
        dx = torch.empty((m, d_in), dtype=torch.float32, device=x.device)
    _shape(dx, (m, d_in), "dx")
    args = [npaths, _dev(bits_u, torch.int32, "bits_u"), _dev(bits_v, torch.int32, "bits_v"),
            _dev(h, torch.float32, "h"), _dev(l, torch.float32, "l"), _dev(g, torch.float32, "g"),
            _dev(x, torch.float32, "x"), _dev(dy, torch.float32, "dy"), _dev(dx, torch.float32, "dx"),
            _dev(dh, torch.float32, "dh"), _dev(dl, torch.float32, "dl"), _dev(dg, torch.float32, "dg"),
            m, d_in, d_out, r, float(gscale)]
    L = lib()
    if saved is not None:
        need = blr_saved_size(npaths, m, d_in, d_out, r)
        if saved.dim() != 1 or saved.numel() < need:
            raise ValueError(f"saved must be a flat uint8 tensor of at least {need} bytes")
        _check(L.blr_backward_paths_saved(*args, _dev(saved, torch.uint8, "saved"), saved.numel(),
                                          _stream(stream)), "blr_backward_paths_saved")
    elif use_ws:
        ws = _workspace(workspace, blr_backward_workspace_size(m, d_in, d_out, r), x, stream,
                        "blr_backward_workspace_size")
        _check(L.blr_backward_paths_ws(*args, _dev(ws, torch.uint8, "workspace"), ws.numel(), _stream(stream)),
               "blr_backward_paths_ws")
    else:
        _check(L.blr_backward_paths(*args, _stream(stream)), "blr_backward_paths")
    return dx


def blr_backward_paths(bits_u, bits_v, h, l, g, x, dy, dh, dl, dg, dx=None, gscale=1024.0, stream=None):
    """Backward of blr_forward_paths on the same x (library-owned workspace): dh [P][d_out],
    dl [P][r] and dg [P][d_in] are accumulated in place; dx [M][d_in] is overwritten (returned)."""
    return _blr_backward_call(bits_u, bits_v, h, l, g, x, dy, dh, dl, dg, dx, gscale, stream, None, False)


def blr_backward_paths_ws(bits_u, bits_v, h, l, g, x, dy, dh, dl, dg, dx=None, gscale=1024.0, workspace=None,
                          stream=None):
    """blr_backward_paths with a caller-owned workspace (uint8, >= blr_backward_workspace_size bytes)."""
    return _blr_backward_call(bits_u, bits_v, h, l, g, x, dy, dh, dl, dg, dx, gscale, stream, workspace, True)
