"""GPU parity of the binary low-rank backward (blr_backward_paths) with the oracle.

The backward of "cortiq-engine 0.8.43 -- train_mm.rs" (module header; blr_backward):
per path dh = sum_t dy.c, db = (dy.h) S_U, dl = sum_t a.db, dx' = (db.l) S_V^T,
dg = sum_t x.dx', and dx = sum_p g.dx', with the products' inputs staged in f16
under a power-of-two gradient scale.  The page's own bar (blr_layer_matches_host):
relative Frobenius error < 3e-3 for dx and for every path's dh, dl and dg against
the f64 reference.  Beyond that: bitwise determinism, exact accumulation into the
gradient buffers, and the layer's dx composed from single-path runs to the bit.
"""

import numpy as np
import pytest

import bit_weight_gemm_amd as bw
import oracle
import workloads as wl
from gpu_util import bits_dev, note, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _stack(paths, key):
    return np.ascontiguousarray(np.stack([p[key] for p in paths]))


def _run(paths, x, dy, gscale, grads=None):
    """(dx, dh, dl, dg) from the GPU; the gradient buffers start at `grads` (zeros)."""
    torch = torch_cuda()
    m, d_in = x.shape
    npaths, d_out, r = len(paths), paths[0]["h"].size, paths[0]["l"].size
    if grads is None:
        grads = [torch.zeros((npaths, n), device="cuda") for n in (d_out, r, d_in)]
    base = torch.full((m * d_in + 64,), float("nan"), device="cuda")
    dx = base[: m * d_in].view(m, d_in)
    bw.blr_backward_paths(bits_dev(_stack(paths, "bits_u")), bits_dev(_stack(paths, "bits_v")),
                          to_dev(_stack(paths, "h")), to_dev(_stack(paths, "l")), to_dev(_stack(paths, "g")),
                          to_dev(x), to_dev(dy), *grads, dx=dx, gscale=gscale)
    torch.cuda.synchronize()
    assert np.isnan(base[m * d_in:].cpu().numpy()).all(), "write past the end of dx"
    out = dx.cpu().numpy()
    assert not np.isnan(out).any(), "unwritten dx"
    return out, [gr.cpu().numpy() for gr in grads], grads


def _rel(got, want):
    want = np.asarray(want, dtype=np.float64)
    num = np.sum((np.asarray(got, dtype=np.float64) - want) ** 2)
    return float(np.sqrt(num / max(np.sum(want ** 2), 1e-300)))


def _check(paths, x, dy, gscale, what):
    note(f"[blr backward {what}] paths={len(paths)} M={x.shape[0]} d_in={x.shape[1]} "
         f"d_out={paths[0]['h'].size} r={paths[0]['l'].size}")
    dx, (dh, dl, dg), _ = _run(paths, x, dy, gscale)
    dx64, grads64 = oracle.blr_backward_paths(paths, x, dy)
    errs = {"dx": _rel(dx, dx64)}
    for p, (h64, l64, g64) in enumerate(grads64):
        errs[f"dh{p}"] = _rel(dh[p], h64)
        errs[f"dl{p}"] = _rel(dl[p], l64)
        errs[f"dg{p}"] = _rel(dg[p], g64)
    note("  " + ", ".join(f"{k} {v:.2g}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v < 3e-3, (what, k, v)


def _page_layer(npaths=2, ntok=70):
    paths = [wl.blr_page_inputs(path=p, ntok=ntok) for p in range(npaths)]
    x = paths[0]["x"]
    for p in paths:
        p.pop("x")
    dy = wl.xorshift_rnd(ntok * 256, 61, 1e-3).reshape(ntok, 256)
    return paths, x, dy


def test_blr_backward_trainer_layer(torch):
    """The page's two-path layer test: m=256, n=384, r=128, 70 tokens, dy in [-1e-3, 1e-3],
    gradient scale 1024."""
    paths, x, dy = _page_layer()
    _check(paths, x, dy, 1024.0, "trainer layer")


def _paths(m, d_in, d_out, r, npaths, index):
    paths = [wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=index + p) for p in range(npaths)]
    x = paths[0]["x"]
    for p in paths:
        p.pop("x")
    dy = (np.random.default_rng(index).standard_normal((m, d_out)) * 1e-3).astype(np.float32)
    return paths, x, dy


@pytest.mark.parametrize("m,d_in,d_out,r,npaths", [(1, 64, 64, 32, 1), (70, 45, 130, 96, 2), (3, 1000, 24, 64, 1),
                                                   (129, 256, 77, 160, 3), (200, 64, 64, 32, 1)])
def test_blr_backward_ragged_shapes(torch, m, d_in, d_out, r, npaths):
    paths, x, dy = _paths(m, d_in, d_out, r, npaths, 40 + m)
    _check(paths, x, dy, 1024.0, f"ragged {m}x{d_in}x{d_out}x{r}")


def test_blr_backward_full_size(torch):
    """The forward's workload (M=512, d_in=d_out=4096, r=1024), dy ~ 1e-3 N(0, 1)."""
    paths, x, dy = _paths(512, 4096, 4096, 1024, 1, 4)
    _check(paths, x, dy, 1024.0, "M=512 d=4096 r=1024")


def test_blr_backward_accumulates_and_repeats_bitwise(torch):
    """A second call on the same buffers adds the same sums (dh = s + s = 2s exactly)
    and overwrites dx with the same bits."""
    paths, x, dy = _paths(70, 45, 130, 96, 2, 7)
    dx1, (dh1, dl1, dg1), grads = _run(paths, x, dy, 256.0)
    dx2, (dh2, dl2, dg2), _ = _run(paths, x, dy, 256.0, grads=grads)
    assert np.array_equal(dx1.view(np.uint32), dx2.view(np.uint32))
    for a, b in ((dh1, dh2), (dl1, dl2), (dg1, dg2)):
        assert np.array_equal((2 * a).view(np.uint32), b.view(np.uint32))


def test_blr_backward_paths_compose_bitwise(torch):
    """dx of a two-path layer is the two single-path dx added in f32, to the bit, and
    each path's gradients are that path's alone."""
    paths, x, dy = _paths(70, 45, 130, 96, 2, 9)
    dx, (dh, dl, dg), _ = _run(paths, x, dy, 1024.0)
    dx0, g0, _ = _run(paths[:1], x, dy, 1024.0)
    dx1, g1, _ = _run(paths[1:], x, dy, 1024.0)
    assert np.array_equal(dx.view(np.uint32), (dx0 + dx1).astype(np.float32).view(np.uint32))
    for k, (a, b) in enumerate(zip((dh, dl, dg), zip(g0, g1))):
        assert np.array_equal(a[0].view(np.uint32), b[0][0].view(np.uint32)), k
        assert np.array_equal(a[1].view(np.uint32), b[1][0].view(np.uint32)), k


def test_blr_backward_rejects_bad_gradient_scale(torch):
    paths, x, dy = _paths(4, 64, 64, 32, 1, 3)
    with pytest.raises(bw.Tq2Error):
        _run(paths, x, dy, 3.0)
    with pytest.raises(bw.Tq2Error):
        _run(paths, x, dy, 0.0)


def test_blr_backward_rejects_misaligned_and_overlapping_buffers(torch):
    """l must be 16-byte aligned; dx must not overlap dy or another output."""
    paths, x, dy = _paths(4, 64, 64, 32, 1, 5)
    d = paths[0]
    bu, bv = bits_dev(d["bits_u"][None]), bits_dev(d["bits_v"][None])
    h, g = to_dev(d["h"][None]), to_dev(d["g"][None])
    xd, dyd = to_dev(x), to_dev(dy)
    grads = [torch.zeros((1, n), device="cuda") for n in (64, 32, 64)]
    l_store = torch.zeros(33 + 3, device="cuda")
    l_bad = l_store[1:33].view(1, 32)            # 4-byte but not 16-byte aligned
    l_bad.copy_(to_dev(d["l"][None]))
    with pytest.raises(bw.Tq2Error):
        bw.blr_backward_paths(bu, bv, h, l_bad, g, xd, dyd, *grads)
    l_ok = to_dev(d["l"][None])
    shared = torch.zeros(4 * 64, device="cuda")
    with pytest.raises(bw.Tq2Error):              # dx on top of dy
        bw.blr_backward_paths(bu, bv, h, l_ok, g, xd, shared.view(4, 64), *grads, dx=shared.view(4, 64))
    with pytest.raises(bw.Tq2Error):              # dh on top of dg
        both = torch.zeros(64, device="cuda")
        bw.blr_backward_paths(bu, bv, h, l_ok, g, xd, dyd, both.view(1, 64), grads[1], both.view(1, 64))
    torch.cuda.synchronize()
