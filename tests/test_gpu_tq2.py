"""GPU parity of the ternary GEMM (tq2_upload / tq2_gemm / tq2_dequant) with the oracle.

Tolerances (per output, against the oracle's f64 value and its bound
B = sum_k |x*w|): f32 path 1e-5*B, f16 MFMA path 4e-3*B; on the tiny workload
the f32 path also meets the correctness test's 1e-3 absolute bar ("oxibonsai-
kernels 0.2.1 -- tests_gemm_tq2.rs", test_encode_gemm_tq2_matches_reference).
"""

import json
import os
import struct

import numpy as np
import pytest

import bit_weight_gemm_amd as bw
import oracle
import workloads as wl
from gpu_util import (F32_REL, MFMA_REL, assert_within, check_tq2_full, check_tq2_sampled, note, run_tq2,
                      to_dev, torch_cuda)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _dequant_gpu(aos, n, k):
    torch = torch_cuda()
    w = bw.tq2_upload(aos, n, k)
    try:
        base = torch.full((n * k + 16,), float("nan"), device="cuda")
        out = base[: n * k].view(n, k)
        bw.tq2_dequant(w, out)
        torch.cuda.synchronize()
        assert np.isnan(base[n * k:].cpu().numpy()).all()
        return out.cpu().numpy()
    finally:
        w.close()


def test_dequant_bit_exact_golden_blocks(torch):
    g = json.load(open(os.path.join(GOLDEN, "tq2_decode_blocks.json")))
    raw = b""
    for case in g["cases"]:
        b = bytearray([int(case["fill"], 16)] * 32)
        for i, v in case["bytes"].items():
            b[int(i)] = int(v, 16)
        raw += bytes(b) + struct.pack("<H", int(case["d"], 16))
    aos = np.frombuffer(raw, np.uint8)
    n = len(g["cases"])
    note("[dequant] golden blocks")
    got = _dequant_gpu(aos, n, 128)
    want = oracle.dequant(aos, n, 128)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("n,k", [(40, 256), (300, 3072), (1, 128)])
def test_dequant_bit_exact_random(torch, n, k):
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 4, (n, k)).astype(np.uint8)          # includes code 3
    bits = rng.integers(0, 0x7C00, (n, k // 128)).astype(np.uint16)  # finite, subnormals included
    bits |= (rng.integers(0, 2, bits.shape) << 15).astype(np.uint16)  # negative scales too
    aos = wl.pack_tq2_aos(codes, bits)
    note(f"[dequant] random n={n} k={k}")
    got = _dequant_gpu(aos, n, k)
    want = oracle.dequant(aos, n, k)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("path", ["f32", "mfma"])
@pytest.mark.parametrize("m", wl.TINY_MS)
def test_tiny_workload(torch, m, path):
    aos, n, k = wl.tiny_weight()
    check_tq2_full(aos, n, k, wl.tiny_x(m, k), path, f"tiny M={m}", page_abs=(path == "f32"))


def test_tiny_workload_auto_path(torch):
    aos, n, k = wl.tiny_weight()
    for m in wl.TINY_MS:
        path = "f32" if bw.tq2_select_path(m) == bw.TQ2_PATH_F32 else "mfma"
        w = bw.tq2_upload(aos, n, k)
        try:
            x = to_dev(wl.tiny_x(m, k))
            y = bw.tq2_gemm(w, x).cpu().numpy()
        finally:
            w.close()
        y64, b = oracle.gemm(aos, n, k, wl.tiny_x(m, k))
        assert_within(y, y64, b, F32_REL if path == "f32" else MFMA_REL, f"tiny auto M={m} ({path})")


SWEEP = [(n, k) for n in wl.SWEEP_NS for k in wl.SWEEP_KS]


@pytest.mark.parametrize("path", ["f32", "mfma"])
@pytest.mark.parametrize("n,k", SWEEP)
def test_parity_sweep(torch, n, k, path):
    """The page's sweep M x N x K, including non-tile multiples (N=40, M=33, M=100)."""
    aos = wl.sweep_weight(n, k)
    w = bw.tq2_upload(aos, n, k)
    try:
        for m in wl.SWEEP_MS:
            x = wl.sweep_x(m, k)
            if m * n * k <= 200_000_000:
                note(f"[sweep] M={m} N={n} K={k} {path}")
                y = run_tq2(w, x, path)
                y64, b = oracle.gemm(aos, n, k, x)
                assert_within(y, y64, b, F32_REL if path == "f32" else MFMA_REL, f"sweep M={m} N={n} K={k}")
                y32 = oracle.gemm_f32seq(aos, n, k, x) if m * n * k <= 20_000_000 else None
                if path == "f32" and y32 is not None:
                    assert np.max(np.abs(y - y32)) < 1e-3
            else:
                check_tq2_sampled(aos, n, k, x, path, f"sweep M={m} N={n} K={k}", w=w)
    finally:
        w.close()


@pytest.mark.parametrize("path", ["f32", "mfma"])
def test_decode_gemv_full(torch, path):
    aos, x = wl.decode_inputs()
    check_tq2_full(aos, 4096, 4096, x, path, "decode M=1")


@pytest.mark.parametrize("path", ["f32", "mfma"])
@pytest.mark.parametrize("m", [8, 32])
def test_mlp_full(torch, m, path):
    aos, x = wl.mlp_inputs(m)
    check_tq2_full(aos, 14336, 4096, x, path, f"mlp M={m}")


@pytest.mark.parametrize("path", ["mfma", "f32"])
def test_prefill_sampled(torch, path):
    aos, x = wl.prefill_inputs()
    check_tq2_sampled(aos, 4096, 4096, x, path, "prefill M=2048", count=4096)


DIT_SHAPES = list(wl.DIT_SHAPES)


@pytest.mark.parametrize("path", ["f32", "mfma"])
@pytest.mark.parametrize("m,n,k", DIT_SHAPES)
def test_dit_shapes_sampled(torch, m, n, k, path):
    """The DiT benchmark shapes of "oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs" (LCG
    weights, scale 0.0625): K = 3072 is 24 blocks, and 1536 x 3072 gives fewer 128 x 256
    tiles than the chip has CUs."""
    aos, x = wl.dit_weight(n, k), wl.dit_x(m, k)
    check_tq2_sampled(aos, n, k, x, path, f"DiT {m}x{n}x{k}", count=4096)


def test_results_are_deterministic(torch):
    aos, x = wl.mlp_inputs(32)
    w = bw.tq2_upload(aos, 14336, 4096)
    try:
        for path in ("f32", "mfma"):
            a = run_tq2(w, x, path)
            b = run_tq2(w, x, path)
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), path
    finally:
        w.close()


@pytest.mark.parametrize("path", ["f32", "mfma"])
@pytest.mark.parametrize("n,k", [(77, 384), (77, 512), (1, 4096), (259, 1024)])
def test_odd_widths(torch, n, k, path):
    """N not a multiple of 4 (padded row quads) and a single output row, at M from 1 to
    past the small-M kernels (M=100), full comparison with the oracle."""
    aos = wl.sweep_weight(n, k)
    w = bw.tq2_upload(aos, n, k)
    try:
        for m in (1, 3, 8, 17, 33, 100):
            x = wl.sweep_x(m, k)
            note(f"[odd widths] M={m} N={n} K={k} {path}")
            y = run_tq2(w, x, path)
            y64, b = oracle.gemm(aos, n, k, x)
            assert_within(y, y64, b, F32_REL if path == "f32" else MFMA_REL, f"odd widths M={m} N={n} K={k}")
    finally:
        w.close()


@pytest.mark.parametrize("n,k", [(600, 768), (600, 640)])
def test_large_m_tile_boundaries(torch, n, k):
    """M just past the small-M kernels and around the 96- and 128-row tiles the MFMA
    path picks for M > 64 (rows past M read row M-1 and are not stored), N = 600
    (a ragged third column tile), K/128 = 6 (two k groups splitting the partial-tile
    sums) and 5 (one k group); full comparison with the oracle and a bitwise repeat."""
    aos = wl.sweep_weight(n, k)
    w = bw.tq2_upload(aos, n, k)
    try:
        for m in (65, 95, 96, 97, 127, 128, 129, 191, 192, 193):
            x = wl.sweep_x(m, k)
            note(f"[large-M tiles] M={m} N={n} K={k}")
            y = run_tq2(w, x, "mfma")
            y64, b = oracle.gemm(aos, n, k, x)
            assert_within(y, y64, b, MFMA_REL, f"large-M tiles M={m} N={n} K={k}")
            again = run_tq2(w, x, "mfma")
            assert np.array_equal(y.view(np.uint32), again.view(np.uint32)), f"not deterministic at M={m}"
    finally:
        w.close()


def test_x_beyond_2gb_uses_64bit_addresses(torch):
    """x of more than 2 GB (130944 x 4096 f32): the large-M tiles read it with 64-bit
    addresses instead of the 32-bit buffer offsets used below 2 GB; sampled outputs
    across the whole range of rows against the oracle."""
    n, k, m = 64, 4096, 130944
    assert (m + 256) * k * 4 >= 2 ** 31
    aos = wl.sweep_weight(n, k)
    x = wl.sweep_x(m, k)
    check_tq2_sampled(aos, n, k, x, "mfma", "x beyond 2 GB", count=2048)


@pytest.mark.parametrize("n,k", [(1000, 4096), (1000, 4608), (5000, 4096)])
def test_f32_path_up_to_four_rows(torch, n, k):
    """M = 1..4 on the f32 path: all activation rows in one launch with four weight rows
    per lane (N = 1000, a ragged last workgroup; K = 4608 takes a second, partial
    4096-wide pass), or eight weight rows per lane (N = 5000, past 4096 rows, for
    M = 2..4). Full comparison with the oracle at the f32 bound; with four rows per lane,
    M = 2..4 give each row's bits of the M = 1 call on that row alone."""
    aos = wl.sweep_weight(n, k)
    w = bw.tq2_upload(aos, n, k)
    try:
        x4 = wl.sweep_x(4, k)
        singles = [run_tq2(w, x4[i:i + 1].copy(), "f32") for i in range(4)]
        for m in (1, 2, 3, 4):
            note(f"[f32 M<=4] M={m} N={n} K={k}")
            x = x4[:m].copy()
            y = run_tq2(w, x, "f32")
            y64, b = oracle.gemm(aos, n, k, x)
            assert_within(y, y64, b, F32_REL, f"f32 M={m} N={n} K={k}")
            if n <= 4096:
                for i in range(m):
                    assert np.array_equal(y[i].view(np.uint32), singles[i][0].view(np.uint32)), f"row {i} of M={m}"
    finally:
        w.close()


@pytest.mark.parametrize("path", ["f32", "mfma"])
def test_many_rows(torch, path):
    """M = 300000 rows: the f32 path's grid runs in slices of 65535 row tiles, and the
    MFMA path has 2344 row tiles; sampled outputs across every slice against the oracle."""
    aos, n, k = wl.tiny_weight()
    x = wl.sweep_x(300000, k)
    check_tq2_sampled(aos, n, k, x, path, "M=300000", count=4096)


def test_zero_rows_is_a_noop(torch):
    aos, n, k = wl.tiny_weight()
    w = bw.tq2_upload(aos, n, k)
    try:
        x = torch.empty((0, k), device="cuda")
        y = torch.empty((0, n), device="cuda")
        for path in (bw.TQ2_PATH_AUTO, bw.TQ2_PATH_F32, bw.TQ2_PATH_MFMA):
            bw.tq2_gemm_path(w, x, y, path)
        torch.cuda.synchronize()
    finally:
        w.close()


def test_argument_errors(torch):
    import ctypes

    L = bw.lib()
    aos, n, k = wl.tiny_weight()
    w = bw.tq2_upload(aos, n, k)
    try:
        x = torch.zeros((4, k), device="cuda")
        y = torch.zeros((4, n), device="cuda")
        xp, yp = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr())
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert L.tq2_gemm(w.handle, xp, yp, 4, n + 1, k, s) == bw.TQ2_EINVAL          # N mismatch
        assert L.tq2_gemm(w.handle, xp, yp, 4, n, k + 128, s) == bw.TQ2_EINVAL        # K mismatch
        assert L.tq2_gemm(w.handle, ctypes.c_void_p(x.data_ptr() + 4), yp, 4, n, k, s) == bw.TQ2_EINVAL
        assert L.tq2_gemm(w.handle, xp, ctypes.c_void_p(y.data_ptr() + 8), 4, n, k, s) == bw.TQ2_EINVAL
        assert L.tq2_gemm(w.handle, xp, xp, 4, n, k, s) == bw.TQ2_EINVAL             # y overlaps x
        assert L.tq2_gemm(w.handle, None, yp, 4, n, k, s) == bw.TQ2_EINVAL
        assert L.tq2_gemm(None, xp, yp, 4, n, k, s) == bw.TQ2_EINVAL
        assert L.tq2_gemm_path(w.handle, xp, yp, 4, n, k, 7, s) == bw.TQ2_EINVAL
        assert L.tq2_dequant(w.handle, ctypes.c_void_p(y.data_ptr() + 4), s) == bw.TQ2_EINVAL
        torch.cuda.synchronize()
        assert np.all(y.cpu().numpy() == 0.0)  # nothing was launched
    finally:
        w.close()


def test_non_finite_scale_is_rejected(torch):
    codes = np.ones((2, 128), np.uint8)
    for bad in (0x7C00, 0xFC00, 0x7E00):
        aos = wl.pack_tq2_aos(codes, np.array([[0x3C00], [bad]], np.uint16))
        with pytest.raises(bw.Tq2Error):
            bw.tq2_upload(aos, 2, 128)


def test_code3_with_huge_scale_uses_exact_path(torch):
    """2d beyond f16 cannot be an MFMA operand; a forced MFMA call must still be exact."""
    codes = np.full((3, 256), 1, np.uint8)
    codes[1, 7] = 3
    codes[2, 200] = 2
    bits = wl.f16_bits(np.array([[1.0, 2.0], [40000.0, 0.5], [0.25, 60000.0]]))
    aos = wl.pack_tq2_aos(codes, bits)
    x = np.random.default_rng(1).standard_normal((5, 256)).astype(np.float32)
    y64, b = oracle.gemm(aos, 3, 256, x)
    w = bw.tq2_upload(aos, 3, 256)
    try:
        y = run_tq2(w, x, "mfma")
    finally:
        w.close()
    assert_within(y, y64, b, F32_REL, "code-3 huge scale")
