"""Shared helpers of the GPU parity tests (test infrastructure)."""

from __future__ import annotations

import sys

import numpy as np

import bit_weight_gemm_amd as bw
import oracle

F32_REL = 1e-5      # f32 path: |err| <= 1e-5 * sum_k |x*w| per output
MFMA_REL = 4e-3     # f16 MFMA path: |err| <= 4e-3 * sum_k |x*w| per output
PAGE_ABS = 1e-3     # the tiny workload's absolute bar (ternary-GEMM correctness test)

PATHS = {"f32": bw.TQ2_PATH_F32, "mfma": bw.TQ2_PATH_MFMA}


def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    return torch


def note(msg: str):
    """Print and flush what the next GPU step is, so a dying run names its case."""
    print(msg, file=sys.stderr, flush=True)


def to_dev(a, dtype=None):
    torch = torch_cuda()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bits_dev(bits):
    return to_dev(np.ascontiguousarray(bits, np.uint32).view(np.int32))


def sample_indices(m: int, n: int, count: int, seed: int = 0):
    """Sampled (m, n) pairs: random ones plus the corners and the last row/column."""
    rng = np.random.default_rng(seed)
    mi = list(rng.integers(0, m, count))
    ni = list(rng.integers(0, n, count))
    for a, b in [(0, 0), (0, n - 1), (m - 1, 0), (m - 1, n - 1)]:
        mi.append(a)
        ni.append(b)
    for j in range(min(n, 64)):
        mi.append(m - 1)
        ni.append(n - 1 - j)
    return np.array(mi, np.int64), np.array(ni, np.int64)


def assert_within(got, want, bound, rel, what):
    got = np.asarray(got, np.float64)
    err = np.abs(got - want)
    tol = rel * np.asarray(bound)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs outside {rel:g}*bound; first at {tuple(i)}: "
                             f"got {got[tuple(i)]!r} want {want[tuple(i)]!r} bound {bound[tuple(i)]!r}")
    ratio = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    note(f"  {what}: max err/tol = {ratio:.3g}")
    return ratio


def run_tq2(w, x_np, path, poison=True):
    """Run tq2_gemm_path on device copies; y starts as NaN so unwritten outputs show."""
    torch = torch_cuda()
    x = to_dev(x_np)
    m = x_np.shape[0]
    base = torch.full((m * w.N + 64,), float("nan"), dtype=torch.float32, device="cuda")
    y = base[: m * w.N].view(m, w.N)
    bw.tq2_gemm_path(w, x, y, PATHS[path] if isinstance(path, str) else path)
    torch.cuda.synchronize()
    tail = base[m * w.N:].cpu().numpy()
    assert np.isnan(tail).all(), "write past the end of y"
    return y.cpu().numpy()


def check_tq2_full(aos, n, k, x_np, path, what, page_abs=False):
    """Element-by-element parity with the oracle over the whole output."""
    w = bw.tq2_upload(aos, n, k)
    try:
        note(f"[tq2 {what}] M={x_np.shape[0]} N={n} K={k} path={path}")
        y = run_tq2(w, x_np, path)
    finally:
        w.close()
    assert not np.isnan(y).any(), f"{what}: unwritten outputs"
    y64, b = oracle.gemm(aos, n, k, x_np)
    rel = F32_REL if path == "f32" else MFMA_REL
    assert_within(y, y64, b, rel, f"{what} {path}")
    if page_abs:
        y32 = oracle.gemm_f32seq(aos, n, k, x_np)
        assert np.max(np.abs(y - y32)) < PAGE_ABS, f"{what}: page's 1e-3 bar vs its f32 reference"
        assert np.max(np.abs(y - y64)) < PAGE_ABS
    if y.size:
        assert np.any(np.abs(y) > 1e-6), f"{what}: output all zero"
    return y


def check_tq2_sampled(aos, n, k, x_np, path, what, count=2048, w=None, y=None):
    """Parity on sampled outputs (full-size workloads)."""
    own = w is None
    if own:
        w = bw.tq2_upload(aos, n, k)
    try:
        if y is None:
            note(f"[tq2 {what}] M={x_np.shape[0]} N={n} K={k} path={path} (sampled)")
            y = run_tq2(w, x_np, path)
    finally:
        if own:
            w.close()
    assert not np.isnan(y).any(), f"{what}: unwritten outputs"
    mi, ni = sample_indices(x_np.shape[0], n, count)
    y64, b = oracle.gemm_at(aos, n, k, x_np, mi, ni)
    rel = F32_REL if path == "f32" else MFMA_REL
    assert_within(y[mi, ni], y64, b, rel, f"{what} {path} sampled")
    return y
