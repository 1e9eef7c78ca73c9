"""GPU checks of the layer forward that keeps its activations and of the backward
that reads them (blr_forward_paths_save, blr_backward_paths_saved).

"cortiq-engine 0.8.43 -- train_mm.rs", blr_forward / blr_backward: the forward
keeps each path's a and c in its scratch and the backward reads them.  Here the
saved values must be the forward's own (y bitwise equal to blr_forward_paths, a
and c against the f64 oracle), and the backward from them must give the bits of
the recomputing backward (blr_backward_paths) and the page's relative bar
against the oracle.
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


def _layer(m, d_in, d_out, r, npaths, index):
    paths = [wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=index + p) for p in range(npaths)]
    x = paths[0]["x"]
    for p in paths:
        p.pop("x")
    dy = (np.random.default_rng(index).standard_normal((m, d_out)) * 1e-3).astype(np.float32)
    return paths, x, dy


def _dev_layer(paths):
    st = lambda key: np.ascontiguousarray(np.stack([p[key] for p in paths]))  # noqa: E731
    return (bits_dev(st("bits_u")), bits_dev(st("bits_v")), to_dev(st("h")), to_dev(st("l")), to_dev(st("g")))


def _rel(got, want):
    want = np.asarray(want, dtype=np.float64)
    return float(np.sqrt(np.sum((np.asarray(got, np.float64) - want) ** 2) / max(np.sum(want ** 2), 1e-300)))


def _bits_equal(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


# the last two: the first product's contraction split over workgroups (two chunks, two paths), and not
SHAPES = [(1, 64, 64, 32, 1), (70, 45, 130, 96, 2), (129, 256, 77, 160, 3), (300, 4096, 200, 1024, 2),
          (512, 4096, 4096, 1024, 1)]


@pytest.mark.parametrize("m,d_in,d_out,r,npaths", SHAPES)
def test_saved_forward_and_backward(torch, m, d_in, d_out, r, npaths):
    note(f"[blr saved] paths={npaths} M={m} d_in={d_in} d_out={d_out} r={r}")
    paths, x, dy = _layer(m, d_in, d_out, r, npaths, 60 + m)
    bu, bv, h, l, g = _dev_layer(paths)
    xd, dyd = to_dev(x), to_dev(dy)
    # the forward: y with the bits of blr_forward_paths; a and c kept per path
    y_ref = bw.blr_forward_paths(bu, bv, h, l, g, xd).cpu().numpy()
    need = bw.blr_saved_size(npaths, m, d_in, d_out, r)
    saved = torch.full((need + 256,), 0xAB, dtype=torch.uint8, device="cuda")
    y, _ = bw.blr_forward_paths_save(bu, bv, h, l, g, xd, saved=saved[:need])
    torch.cuda.synchronize()
    assert _bits_equal(y.cpu().numpy(), y_ref), "saving changes y"
    assert (saved[need:].cpu().numpy() == 0xAB).all(), "write past the end of the saved buffer"
    for p, (a, c) in enumerate(bw.blr_saved_views(saved, npaths, m, d_out, r)):
        y64, a64 = oracle.blr_forward(x=x, want_a=True, **paths[p])
        assert _rel(a.cpu().numpy(), a64) < 3e-3, f"path {p}: a"
        assert _rel(c.cpu().numpy(), y64 / paths[p]["h"][None, :].astype(np.float64)) < 3e-3, f"path {p}: c"
        # c = y_p / h_p in exact arithmetic: compare h*c with the path's own forward
        yp = bw.blr_forward(*(t[p] for t in (bu, bv, h, l, g)), xd).cpu().numpy()
        hc = (paths[p]["h"][None, :] * c.cpu().numpy()).astype(np.float32)
        assert _bits_equal(hc, yp), f"path {p}: h*c is not the path's own forward"
    # the backward from the saved activations: the recomputing backward's bits
    grads_s = [torch.zeros((npaths, n), device="cuda") for n in (d_out, r, d_in)]
    grads_r = [torch.zeros((npaths, n), device="cuda") for n in (d_out, r, d_in)]
    dx_s = bw.blr_backward_paths_saved(bu, bv, h, l, g, xd, dyd, *grads_s, saved=saved[:need], gscale=1024.0)
    dx_r = bw.blr_backward_paths(bu, bv, h, l, g, xd, dyd, *grads_r, gscale=1024.0)
    torch.cuda.synchronize()
    assert _bits_equal(dx_s.cpu().numpy(), dx_r.cpu().numpy()), "dx"
    for k, (a, b) in enumerate(zip(grads_s, grads_r)):
        assert _bits_equal(a.cpu().numpy(), b.cpu().numpy()), ("dh", "dl", "dg")[k]
    # and the page's bar against the f64 oracle
    dx64, grads64 = oracle.blr_backward_paths(paths, x, dy)
    assert _rel(dx_s.cpu().numpy(), dx64) < 3e-3
    for p, (h64, l64, g64) in enumerate(grads64):
        for got, want in zip((t[p].cpu().numpy() for t in grads_s), (h64, l64, g64)):
            assert _rel(got, want) < 3e-3


def test_saved_buffer_checks(torch):
    """Too small, misaligned or overlapping saved buffers are refused on the host."""
    paths, x, dy = _layer(4, 64, 64, 32, 1, 3)
    bu, bv, h, l, g = _dev_layer(paths)
    xd, dyd = to_dev(x), to_dev(dy)
    need = bw.blr_saved_size(1, 4, 64, 64, 32)
    big = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    L = bw.lib()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    y = torch.empty((4, 64), device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [1, p(bu), p(bv), p(h), p(l), p(g), p(xd), p(y), 4, 64, 64, 32]
    assert L.blr_forward_paths_save(*args, p(big), need - 1, s) == bw.TQ2_EINVAL          # too small
    assert L.blr_forward_paths_save(*args, p(big[16:]), need, s) == bw.TQ2_EINVAL          # not 256-byte aligned
    ybig = torch.zeros(need // 4 + 64 * 4, device="cuda")
    args_y = [1, p(bu), p(bv), p(h), p(l), p(g), p(xd), p(ybig), 4, 64, 64, 32]
    assert L.blr_forward_paths_save(*args_y, p(ybig), need, s) == bw.TQ2_EINVAL            # saved on top of y
    assert L.blr_forward_paths_save(*args, p(big), need, s) == bw.TQ2_OK
    grads = [torch.zeros((1, n), device="cuda") for n in (64, 32, 64)]
    dx = torch.empty((4, 64), device="cuda")
    bargs = [1, p(bu), p(bv), p(h), p(l), p(g), p(xd), p(dyd), p(dx), *(p(t) for t in grads), 4, 64, 64, 32,
             ctypes.c_float(1024.0)]
    assert L.blr_backward_paths_saved(*bargs, p(big), need - 1, s) == bw.TQ2_EINVAL
    dx_over = big[:4 * 64 * 4].view(torch.float32).view(4, 64)                              # dx on top of saved
    bargs_o = bargs[:8] + [p(dx_over)] + bargs[9:]
    assert L.blr_backward_paths_saved(*bargs_o, p(big), need, s) == bw.TQ2_EINVAL
    assert L.blr_backward_paths_saved(*bargs, p(big), need, s) == bw.TQ2_OK
    torch.cuda.synchronize()
