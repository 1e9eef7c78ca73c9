"""GPU parity of the binary low-rank forward (blr_forward) with the oracle.

Tolerances ("cortiq-engine 0.8.43 -- train_mm.rs", blr_layer_matches_host, and the
MFMA-path bar): relative Frobenius error < 3e-3 over the whole output, and per
output |err| <= 4e-3 * B with B = sum_j |x_j| |W^_ij| the dense-equivalent bound.
"""

import numpy as np
import pytest

import bit_weight_gemm_amd as bw
import oracle
import workloads as wl
from gpu_util import MFMA_REL, assert_within, bits_dev, note, sample_indices, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _run(d, poison=True):
    torch = torch_cuda()
    m, d_out = d["x"].shape[0], d["h"].size
    base = torch.full((m * d_out + 64,), float("nan"), device="cuda")
    y = base[: m * d_out].view(m, d_out)
    bw.blr_forward(bits_dev(d["bits_u"]), bits_dev(d["bits_v"]), to_dev(d["h"]), to_dev(d["l"]),
                   to_dev(d["g"]), to_dev(d["x"]), y)
    torch.cuda.synchronize()
    assert np.isnan(base[m * d_out:].cpu().numpy()).all(), "write past the end of y"
    out = y.cpu().numpy()
    assert not np.isnan(out).any(), "unwritten outputs"
    return out


def _rel_frob(got, want):
    return float(np.sqrt(np.sum((got - want) ** 2) / max(np.sum(want ** 2), 1e-300)))


def _check(d, what, count=None, rel_frob=3e-3):
    m, d_out = d["x"].shape[0], d["h"].size
    note(f"[blr {what}] M={m} d_in={d['x'].shape[1]} d_out={d_out} r={d['l'].size}")
    y = _run(d)
    y64, _ = oracle.blr_forward(**d)
    e = _rel_frob(y, y64)
    note(f"  {what}: relative Frobenius error {e:.3g}")
    assert e < rel_frob
    if count is None:
        ti = np.repeat(np.arange(m), d_out)
        ii = np.tile(np.arange(d_out), m)
    else:
        ti, ii = sample_indices(m, d_out, count, seed=3)
    b = oracle.blr_bound_at(**d, ti=ti, ii=ii)
    assert_within(y[ti, ii], y64[ti, ii], b, MFMA_REL, what)
    return y, y64


def test_blr_trainer_test_shapes(torch):
    """m=256 outputs, n=384 inputs, r=128, 70 tokens: the trainer's own layer test, one path."""
    for path in (0, 1):
        _check(wl.blr_page_inputs(path=path), f"trainer shapes path {path}")


def test_blr_full_size(torch):
    _check(wl.blr_inputs(), "M=512 d=4096 r=1024", count=512)


@pytest.mark.parametrize("m,d_in,d_out,r", [(1, 64, 64, 32), (70, 45, 130, 96), (3, 1000, 24, 64),
                                            (129, 256, 77, 160), (64, 4096, 512, 1024)])
def test_blr_ragged_shapes(torch, m, d_in, d_out, r):
    _check(wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=20 + m), f"ragged {m}x{d_in}x{d_out}x{r}")


@pytest.mark.parametrize("m,d_in,d_out,r", [(300, 4096, 200, 1024), (520, 4000, 96, 1024), (1024, 4096, 64, 256),
                                            (128, 4096, 300, 1024)])
def test_blr_split_contraction(torch, m, d_in, d_out, r):
    """Sizes whose first product splits d_in over workgroups and adds the chunks' partial
    products in a last launch: two chunks with ragged M and vector x loads; two chunks with a
    d_in tail and scalar x loads; two chunks with r = 256; four chunks."""
    _check(wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=50 + m), f"split {m}x{d_in}x{d_out}x{r}",
           count=2048)


def test_blr_many_tokens(torch):
    """Enough tokens that the first product takes its large tiles (4100 x 1024 outputs)."""
    _check(wl.blr_inputs(m=4100, d_in=256, d_out=96, r=1024, index=41), "many tokens", count=2048)


def _exact_grid(m, d_in, d_out, r, seed):
    """Inputs on which every f16 operand and every f32 partial sum is exact.

    The trainer page's exact-grid construction (blr_sign_flip_exact: powers-of-two
    l and g, x on a 1/8 grid), shrunk so that also a.l fits f16 exactly: with
    |x| <= 1/2, g in {1/2, 1}, l in {1/2, 1, 2} and d_in <= 64, a.l is a multiple of
    1/32 of magnitude <= 64 and c = sum_k f16(a.l) S_U is a multiple of 1/32 below
    2^17, so the GPU result is f32(h*c) with c exact: within 2^-24 |y| of the oracle.
    """
    assert d_in <= 64 and r <= 64
    rng = np.random.default_rng(seed)
    d = wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=seed)
    d["l"] = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), r)
    d["g"] = rng.choice(np.array([0.5, 1.0], np.float32), d_in)
    d["x"] = (rng.integers(-4, 5, (m, d_in)) / 8).astype(np.float32)
    return d


def _assert_exact(y, y64, what):
    err = np.abs(y.astype(np.float64) - y64)
    assert np.all(err <= 2.0 ** -24 * np.abs(y64)), f"{what}: max err {err.max():.3g}"


def test_blr_exact_grid_matches_to_the_last_rounding(torch):
    d = _exact_grid(40, 64, 200, 64, 5)
    y64, _ = oracle.blr_forward(**d)
    _assert_exact(_run(d), y64, "exact grid")


def test_blr_sign_flips_on_the_gpu(torch):
    """Flip single signs of S_U and S_V on the exact grid: the GPU output tracks the
    oracle exactly, and a flip of S_U[i][k] leaves every other column bit-identical
    (pins bit order and orientation of both bitmaps on the device path)."""
    d = _exact_grid(16, 64, 80, 64, 9)
    y0 = _run(d)
    _assert_exact(y0, oracle.blr_forward(**d)[0], "base")
    for (i, k) in [(0, 0), (79, 63), (33, 31), (34, 32)]:
        e = dict(d)
        e["bits_u"] = d["bits_u"].copy()
        e["bits_u"][i, k // 32] ^= np.uint32(1 << (k % 32))
        y1 = _run(e)
        _assert_exact(y1, oracle.blr_forward(**e)[0], f"S_U flip {(i, k)}")
        others = np.ones(80, bool)
        others[i] = False
        assert np.array_equal(y1[:, others].view(np.uint32), y0[:, others].view(np.uint32))
        assert not np.array_equal(y1[:, i], y0[:, i])
    for (j, k) in [(0, 0), (63, 63), (40, 17), (5, 32)]:
        e = dict(d)
        e["bits_v"] = d["bits_v"].copy()
        e["bits_v"][j, k // 32] ^= np.uint32(1 << (k % 32))
        y1 = _run(e)
        _assert_exact(y1, oracle.blr_forward(**e)[0], f"S_V flip {(j, k)}")


def test_blr_zero_tokens_is_a_noop(torch):
    d = wl.blr_inputs(m=1, d_in=64, d_out=64, r=32, index=1)
    y = torch.full((0, 64), 1.0, device="cuda")
    bw.blr_forward(bits_dev(d["bits_u"]), bits_dev(d["bits_v"]), to_dev(d["h"]), to_dev(d["l"]),
                   to_dev(d["g"]), torch.empty((0, 64), device="cuda"), y)
    torch.cuda.synchronize()


def test_blr_deterministic(torch):
    d = wl.blr_inputs(m=100, d_in=512, d_out=384, r=256, index=2)
    a, b = _run(d), _run(d)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _stack(paths, key):
    return np.ascontiguousarray(np.stack([p[key] for p in paths]))


def _run_paths(paths, x):
    torch = torch_cuda()
    m, d_out = x.shape[0], paths[0]["h"].size
    base = torch.full((m * d_out + 64,), float("nan"), device="cuda")
    y = base[: m * d_out].view(m, d_out)
    bw.blr_forward_paths(bits_dev(_stack(paths, "bits_u")), bits_dev(_stack(paths, "bits_v")),
                         to_dev(_stack(paths, "h")), to_dev(_stack(paths, "l")), to_dev(_stack(paths, "g")),
                         to_dev(x), y)
    torch.cuda.synchronize()
    assert np.isnan(base[m * d_out:].cpu().numpy()).all(), "write past the end of y"
    out = y.cpu().numpy()
    assert not np.isnan(out).any(), "unwritten outputs"
    return out


def _page_paths(n_paths):
    paths = [wl.blr_page_inputs(path=p) for p in range(n_paths)]
    x = paths[0].pop("x")
    for p in paths[1:]:
        p.pop("x")
    return paths, x


def test_blr_two_path_layer_matches_oracle(torch):
    """The trainer's two-path layer test ("cortiq-engine 0.8.43 -- train_mm.rs",
    blr_layer_matches_host: m=256, n=384, r=128, 70 tokens, np=2): relative Frobenius
    error < 3e-3 against the f64 sum of the paths, and every output within 4e-3 of the
    summed dense-equivalent bounds."""
    paths, x = _page_paths(2)
    note("[blr paths] two-path trainer layer")
    y = _run_paths(paths, x)
    y64 = oracle.blr_forward_paths(paths, x)
    e = _rel_frob(y, y64)
    note(f"  two paths: relative Frobenius error {e:.3g}")
    assert e < 3e-3
    ti = np.repeat(np.arange(x.shape[0]), y.shape[1])
    ii = np.tile(np.arange(y.shape[1]), x.shape[0])
    b = oracle.blr_paths_bound_at(paths, x, ti, ii)
    assert_within(y[ti, ii], y64[ti, ii], b, MFMA_REL, "two-path layer")


@pytest.mark.parametrize("n_paths,shape", [(2, None), (3, (70, 45, 130, 96)), (3, (512, 4096, 512, 1024))])
def test_blr_paths_round_path_by_path(torch, n_paths, shape):
    """The layer output is the single-path outputs added in f32, path by path, to the
    bit: y = f32(f32(h_0 c_0) + f32(h_1 c_1)) (scale_acc2), then + f32(h_2 c_2)."""
    if shape is None:
        paths, x = _page_paths(n_paths)
    else:
        m, d_in, d_out, r = shape
        paths = [wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=30 + p) for p in range(n_paths)]
        x = paths[0]["x"]
        for p in paths:
            p.pop("x")
    note(f"[blr paths] {n_paths} paths, M={x.shape[0]} d_in={x.shape[1]}")
    y = _run_paths(paths, x)
    want = None
    for p in paths:
        yp = _run(dict(p, x=x))
        want = yp if want is None else (want + yp).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    one = _run_paths(paths[:1], x)
    assert np.array_equal(one.view(np.uint32), _run(dict(paths[0], x=x)).view(np.uint32))
