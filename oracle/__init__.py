"""ctypes wrapper of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg, never by the library package.  It shares nothing with the HIP
path; inputs come from `workloads`, which holds no arithmetic of the method.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc: -O2, no fast-math, no contraction, OpenMP."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", tmp, SRC_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        i64, sz, p = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = ctypes.c_int
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.tq2_oracle_dequant.argtypes = [p, sz, i64, i64, p]
        L.tq2_oracle_gemm.argtypes = [p, sz, i64, i64, p, i64, p, p]
        L.tq2_oracle_gemm_at.argtypes = [p, sz, i64, i64, p, i64, p, p, i64, p, p]
        L.tq2_oracle_gemm_f32seq.argtypes = [p, sz, i64, i64, p, i64, p]
        L.blr_oracle_forward.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, p, p]
        L.blr_oracle_bound_at.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, p, p, i64, p]
        for f in ("tq2_oracle_dequant", "tq2_oracle_gemm", "tq2_oracle_gemm_at",
                  "tq2_oracle_gemm_f32seq", "blr_oracle_forward", "blr_oracle_bound_at"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(ValueError):
    pass


def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")


def threads() -> int:
    return int(lib().oracle_threads())


def set_threads(n: int) -> int:
    """Thread count of later oracle calls (OpenMP); returns the count in force."""
    return int(lib().oracle_set_threads(int(n)))


def half_to_double(bits: int) -> float:
    return float(lib().oracle_half_to_double(bits))


def dequant(aos, n: int, k: int) -> np.ndarray:
    aos = _c(aos, np.uint8)
    w = np.empty((n, k), dtype=np.float32)
    _check(lib().tq2_oracle_dequant(_ptr(aos), aos.size, n, k, _ptr(w)))
    return w


def gemm(aos, n: int, k: int, x):
    """(y64 [M][N] float64, bound [M][N] float64) for y = x @ W^T."""
    aos = _c(aos, np.uint8)
    x = _c(x, np.float32).reshape(-1, k)
    m = x.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    b = np.empty((m, n), dtype=np.float64)
    _check(lib().tq2_oracle_gemm(_ptr(aos), aos.size, n, k, _ptr(x), m, _ptr(y), _ptr(b)))
    return y, b


def gemm_at(aos, n: int, k: int, x, mi, ni):
    """Selected outputs (mi[s], ni[s]): (y64 [S], bound [S])."""
    aos = _c(aos, np.uint8)
    x = _c(x, np.float32)
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    y = np.empty(mi.size, dtype=np.float64)
    b = np.empty(mi.size, dtype=np.float64)
    _check(lib().tq2_oracle_gemm_at(_ptr(aos), aos.size, n, k, _ptr(x), x.shape[0],
                                    _ptr(mi), _ptr(ni), mi.size, _ptr(y), _ptr(b)))
    return y, b


def gemm_f32seq(aos, n: int, k: int, x) -> np.ndarray:
    """The correctness test's f32 sequential-accumulation reference."""
    aos = _c(aos, np.uint8)
    x = _c(x, np.float32)
    y = np.empty((x.shape[0], n), dtype=np.float32)
    _check(lib().tq2_oracle_gemm_f32seq(_ptr(aos), aos.size, n, k, _ptr(x), x.shape[0], _ptr(y)))
    return y


def blr_forward(bits_u, bits_v, h, l, g, x, want_a: bool = False):
    """(y64 [M][d_out], a64 [M][r] or None)."""
    bits_u = _c(bits_u, np.uint32)
    bits_v = _c(bits_v, np.uint32)
    h, l, g, x = (_c(v, np.float32) for v in (h, l, g, x))
    m, d_in = x.shape
    d_out, r = h.size, l.size
    y = np.empty((m, d_out), dtype=np.float64)
    a = np.empty((m, r), dtype=np.float64) if want_a else None
    _check(lib().blr_oracle_forward(_ptr(bits_u), _ptr(bits_v), _ptr(h), _ptr(l), _ptr(g), _ptr(x),
                                    m, d_in, d_out, r, _ptr(y), _ptr(a)))
    return y, a


def blr_bound_at(bits_u, bits_v, h, l, g, x, ti, ii) -> np.ndarray:
    bits_u = _c(bits_u, np.uint32)
    bits_v = _c(bits_v, np.uint32)
    h, l, g, x = (_c(v, np.float32) for v in (h, l, g, x))
    ti = _c(ti, np.int64)
    ii = _c(ii, np.int64)
    m, d_in = x.shape
    b = np.empty(ti.size, dtype=np.float64)
    _check(lib().blr_oracle_bound_at(_ptr(bits_u), _ptr(bits_v), _ptr(h), _ptr(l), _ptr(g), _ptr(x),
                                     m, d_in, h.size, l.size, _ptr(ti), _ptr(ii), ti.size, _ptr(b)))
    return b


def blr_forward_paths(paths, x) -> np.ndarray:
    """y64 of a layer of several paths: the sum over paths, in path order, of each
    path's forward ("cortiq-engine 0.8.43 -- train_mm.rs": a Blr layer is y = sum_p
    W^_p x; the f64 reference of its two-path layer test adds h_p c_p path by path).
    `paths` is a sequence of dicts with bits_u, bits_v, h, l, g."""
    y = None
    for p in paths:
        yp, _ = blr_forward(p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"], x)
        y = yp if y is None else y + yp
    return y


def blr_paths_bound_at(paths, x, ti, ii) -> np.ndarray:
    """Sum over paths of each path's dense-equivalent bound at outputs (ti, ii)."""
    b = None
    for p in paths:
        bp = blr_bound_at(p["bits_u"], p["bits_v"], p["h"], p["l"], p["g"], x, ti, ii)
        b = bp if b is None else b + bp
    return b


def _signs(bits, r) -> np.ndarray:
    """[rows][r] of +1.0 / -1.0 from a sign bitmap: rank k is bit k % 32 of word
    k // 32 of the row, a set bit meaning +1 ("cortiq-engine 0.8.43 -- train_mm.rs",
    expand)."""
    bits = np.asarray(bits, dtype=np.uint32)
    out = np.empty((bits.shape[0], r), dtype=np.float64)
    for k in range(r):
        bit = (bits[:, k // 32] >> np.uint32(k % 32)) & np.uint32(1)
        out[:, k] = np.where(bit == 1, 1.0, -1.0)
    return out


def blr_backward_paths(paths, x, dy):
    """Backward of a layer of paths, f64 ("cortiq-engine 0.8.43 -- train_mm.rs",
    module header; the f64 reference of blr_layer_matches_host).  Per path, with
    a = (x.g) S_V and c = (a.l) S_U^T:
        dh = sum_t dy.c,  db = (dy.h) S_U,  dl = sum_t a.db,
        dx' = (db.l) S_V^T,  dg = sum_t x.dx',  and dx = sum_p g.dx'.
    Returns (dx [M][d_in], [(dh, dl, dg) per path]).  The f16 staging and the
    gradient scale of the GPU path are not part of the definition."""
    x64 = np.asarray(x, dtype=np.float64)
    dy64 = np.asarray(dy, dtype=np.float64)
    dx = np.zeros_like(x64)
    grads = []
    for p in paths:
        r = np.asarray(p["l"]).size
        su = _signs(p["bits_u"], r)   # [d_out][r]
        sv = _signs(p["bits_v"], r)   # [d_in][r]
        h, l, g = (np.asarray(p[k], dtype=np.float64) for k in ("h", "l", "g"))
        a = (x64 * g) @ sv
        c = (a * l) @ su.T
        dh = (dy64 * c).sum(axis=0)
        db = (dy64 * h) @ su
        dl = (a * db).sum(axis=0)
        dxp = (db * l) @ sv.T
        dg = (x64 * dxp).sum(axis=0)
        dx += g * dxp
        grads.append((dh, dl, dg))
    return dx, grads
