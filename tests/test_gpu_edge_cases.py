"""GPU parity of every kernel template on the block format's edge cases.

The format ("oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs", correctness test):
each 128-weight block is 32 bytes of 2-bit codes plus an f16 scale d, and
w = (code - 1) * d.  The weights here (`workloads.edge_weight`) hold, row class
by row class: all-0x55 blocks (every code 1: the weight is zero, so y must be
exactly 0), a single nonzero code in a row (y must be exactly +-d*x, rounded
once on the f32 path; on the MFMA path exactly f16(x)*d, which f32 holds
exactly), all-0x00 blocks (every weight -d), subnormal, large (up to 32752,
where 2d is still a finite f16), negative and zero scales, and code 3 (+2d),
which the page's generator never draws.

Each case lands on one kernel template of the f32 or the MFMA path (the label
names it) and is compared with the oracle over every output at the path's bound:
1e-5 * sum_k |x*w| (f32 path), 4e-3 * sum_k |x*w| (MFMA path).  The prefill and
the smaller DiT shape are also compared in full, not sampled.
"""

import numpy as np
import pytest

import bit_weight_gemm_amd as bw
import oracle
import workloads as wl
from gpu_util import F32_REL, MFMA_REL, assert_within, note, run_tq2, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


# (label: the kernel template the case lands on, path, Ms, N, K)
CASES = [
    ("gemv_mt M=1, a second partial 4096-wide pass", "f32", (1,), 1000, 4608),
    ("gemv_mt M=2..4", "f32", (2, 3, 4), 1000, 1024),
    ("gemv_f32 eight rows per lane, M=2", "f32", (2,), 5000, 1024),
    ("gemv_f32 eight rows per lane, M=3 and forced M=7", "f32", (3, 7), 5000, 1024),
    ("skinny 16x16x32, one column per lane, x all at once (M=16: 32 pieces per thread)", "mfma", (1, 8, 16),
     1000, 4096),
    ("skinny 16x16x32, one column per lane, two passes of eight steps (M=3 step by step)", "mfma", (1, 3, 5),
     1000, 8192),
    ("skinny 16x16x32, two columns per lane (M=3 step by step, M=12 all at once)", "mfma", (3, 12), 6000, 2048),
    ("skinny 16x16x32, four columns per lane, N % 4 == 2", "mfma", (2, 12), 12302, 1024),
    ("skinny 16x16x32, four columns per lane, two and four pieces per step (M=13: two passes)", "mfma", (6, 13),
     12302, 4096),
    ("skinny 16x16x32, two row blocks (M=20: six pieces per step, M=32: eight; two passes)", "mfma", (20, 32),
     12302, 2048),
    ("skinny 16x16x32, two row blocks, one column per lane", "mfma", (17,), 1000, 4096),
    ("skinny 32x32x16, K not a multiple of 1024", "mfma", (4, 12), 1000, 1536),
    ("skinny 16x16x32, K=32768: many passes of the load slots", "mfma", (1, 3, 8, 20), 300, 32768),
    ("skinny 16x16x32, K=8192: two and four passes unrolled", "mfma", (3, 12), 6000, 8192),
    ("gemv_mt, K=32768: eight 4096-wide passes", "f32", (1, 4), 300, 32768),
    ("64x64 tiles, K=32768", "mfma", (40,), 300, 32768),
    ("skinny 16x16x32, two row blocks, two columns per lane", "mfma", (20,), 6000, 4096),
    ("skinny 16x16x32, four columns per lane in one round of 141 workgroups", "mfma", (1, 4, 8, 32), 9000, 4096),
    ("32x64 tiles, four k groups", "mfma", (24,), 1000, 1536),
    ("32x64 tiles, two k groups", "mfma", (24,), 1000, 768),
    ("64x64 tiles, 512-wide steps", "mfma", (40,), 1000, 4096),
    ("64x64 tiles, four stages", "mfma", (40,), 1000, 1536),
    ("64x64 tiles, two k groups", "mfma", (40,), 1000, 768),
    ("32x256 tiles, odd block count", "mfma", (40,), 1000, 384),
    ("96x256 tiles", "mfma", (200,), 1000, 768),
    ("128x256 tiles, one k group, odd block count", "mfma", (200,), 1000, 384),
    ("128x256 tiles, two k groups", "mfma", (1600,), 4096, 768),
]


F16_MIN_NORMAL = 2.0 ** -14


def _x(m, k, seed, path):
    """x ~ N(0, 1) with some exact zeros.  On the MFMA path the relative bound
    presumes every nonzero |x| >= 2^-14, since f16 rounds smaller values as
    subnormals with an absolute error up to 2^-25.  A single-code row's bound is
    one product, so one such x would break it: those few values are set to zero
    here, and test_f16_subnormal_x_meets_the_absolute_bound covers them."""
    x = np.random.default_rng(seed).standard_normal((m, k)).astype(np.float32)
    x[:, ::97] = 0.0
    if path == "mfma":
        x[np.abs(x) < F16_MIN_NORMAL] = 0.0
    return x


def _abs_bound_ok(y, y64, b, wabs, what):
    """|err| <= 4e-3 * B + 2^-25 * sum_k |w|: the MFMA bound with x's f16 rounding error
    taken as max(2^-11 |x|, 2^-25) (relative in the normal range, absolute below)."""
    err = np.abs(y.astype(np.float64) - y64)
    tol = MFMA_REL * b + 2.0 ** -25 * wabs[None, :]
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside the bound"
    note(f"  {what}: max err/tol = {float(np.max(err / np.maximum(tol, 1e-300))):.3g}")


def _scale(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _exact_rows(y, x, codes, bits, path):
    """Rows of class 0 give exactly 0; rows of class 1 exactly the one product."""
    n, k = codes.shape
    cls = np.arange(n) % wl.EDGE_CLASSES
    zero_rows = np.flatnonzero(cls == 0)
    assert np.all(y[:, zero_rows] == 0.0), "all-0x55 rows must give exactly 0"
    xs = x.astype(np.float64) if path == "f32" else x.astype(np.float16).astype(np.float64)
    for row in np.flatnonzero(cls == 1):
        pos = int(np.flatnonzero(codes[row] != 1)[0])
        d = _scale(bits[row, pos // wl.BLOCK])
        want = (float(codes[row, pos]) - 1.0) * d * xs[:, pos]   # exact in f64
        want32 = want.astype(np.float32)                          # one rounding (exact on the MFMA path)
        assert np.array_equal(y[:, row], want32), f"single-code row {row}: {y[:4, row]} vs {want32[:4]}"


@pytest.mark.parametrize("label,path,ms,n,k", CASES, ids=[c[0] for c in CASES])
def test_edge_weights_on_every_kernel(torch, label, path, ms, n, k):
    aos, codes, bits = wl.edge_weight(n, k, seed=n + k)
    w = bw.tq2_upload(aos, n, k)
    try:
        for m in ms:
            x = _x(m, k, m + 7 * k, path)
            note(f"[edge] {label}: M={m} N={n} K={k} {path}")
            y = run_tq2(w, x, path)
            assert not np.isnan(y).any(), "unwritten outputs"
            y64, b = oracle.gemm(aos, n, k, x)
            assert_within(y, y64, b, F32_REL if path == "f32" else MFMA_REL, f"edge {label} M={m}")
            _exact_rows(y, x, codes, bits, path)
    finally:
        w.close()


def test_edge_weights_decode_bit_exact(torch):
    """The GPU decode of the edge weight, bit for bit (sign of zero included)."""
    n, k = 1000, 1536
    aos, _, _ = wl.edge_weight(n, k, seed=3)
    w = bw.tq2_upload(aos, n, k)
    try:
        out = bw.tq2_dequant(w)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
    finally:
        w.close()
    assert np.array_equal(got.view(np.uint32), oracle.dequant(aos, n, k).view(np.uint32))


def test_small_magnitude_x(torch):
    """x ~ 1e-3 N(0, 1): about 5% of the values fall below the f16 normal range.  The f32
    path meets its relative bound; the MFMA path meets 4e-3 * B + 2^-25 * sum_k |w| (its
    bound with the subnormal rounding error of x counted as absolute), on the tiled and
    skinny kernels; rows of more than one nonzero weight stay within 4e-3 * B."""
    n, k = 1000, 4096
    aos, codes, _ = wl.edge_weight(n, k, seed=11)
    wabs = np.abs(oracle.dequant(aos, n, k).astype(np.float64)).sum(axis=1)
    w = bw.tq2_upload(aos, n, k)
    try:
        for m, path in ((8, "mfma"), (40, "mfma"), (200, "mfma"), (1, "f32"), (3, "f32")):
            x = (np.random.default_rng(m).standard_normal((m, k)) * 1e-3).astype(np.float32)
            note(f"[edge] small x M={m} {path}")
            y = run_tq2(w, x, path)
            y64, b = oracle.gemm(aos, n, k, x)
            if path == "f32":
                assert_within(y, y64, b, F32_REL, f"small x M={m}")
            else:
                _abs_bound_ok(y, y64, b, wabs, f"small x M={m}")
                many = (np.arange(n) % wl.EDGE_CLASSES) >= 2   # rows with many nonzero weights
                assert_within(y[:, many], y64[:, many], b[:, many], MFMA_REL, f"small x M={m}, dense rows")
    finally:
        w.close()


def test_f16_subnormal_x_meets_the_absolute_bound(torch):
    """x made only of values below the f16 normal range (|x| < 2^-14): the MFMA path's
    error stays within 4e-3 * B + 2^-25 * sum_k |w| on every kernel family."""
    n, k = 1000, 4096
    aos, _, _ = wl.edge_weight(n, k, seed=12)
    wabs = np.abs(oracle.dequant(aos, n, k).astype(np.float64)).sum(axis=1)
    w = bw.tq2_upload(aos, n, k)
    try:
        for m in (8, 40, 200):
            x = (np.random.default_rng(100 + m).uniform(-1, 1, (m, k)) * F16_MIN_NORMAL).astype(np.float32)
            note(f"[edge] subnormal x M={m}")
            y = run_tq2(w, x, "mfma")
            y64, b = oracle.gemm(aos, n, k, x)
            _abs_bound_ok(y, y64, b, wabs, f"subnormal x M={m}")
    finally:
        w.close()


def test_prefill_full(torch):
    """Every one of the 8.4 M outputs of the 2048 x 4096 x 4096 prefill, both paths."""
    aos, x = wl.prefill_inputs()
    n = k = 4096
    y64, b = oracle.gemm(aos, n, k, x)
    w = bw.tq2_upload(aos, n, k)
    try:
        for path in ("mfma", "f32"):
            note(f"[prefill full] M=2048 N=4096 K=4096 {path}")
            y = run_tq2(w, x, path)
            assert not np.isnan(y).any()
            assert_within(y, y64, b, F32_REL if path == "f32" else MFMA_REL, f"prefill full {path}")
    finally:
        w.close()


def test_dit_small_shape_full(torch):
    """The DiT 1536 x 3072 x 3072 benchmark shape ("oxibonsai-kernels 0.2.1 --
    tests_gemm_tq2.rs", DiT benchmarks), every output, both paths."""
    m, n, k = 1536, 3072, 3072
    aos, x = wl.dit_weight(n, k), wl.dit_x(m, k)
    y64, b = oracle.gemm(aos, n, k, x)
    w = bw.tq2_upload(aos, n, k)
    try:
        for path in ("mfma", "f32"):
            note(f"[DiT full] {m}x{n}x{k} {path}")
            y = run_tq2(w, x, path)
            assert_within(y, y64, b, F32_REL if path == "f32" else MFMA_REL, f"DiT full {path}")
    finally:
        w.close()
