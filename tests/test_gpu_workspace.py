"""The library's workspaces are grow-only and allocated once per (device, stream).

"oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs", pool tests: after a warm-up at the
largest size, later GEMM calls must not add device allocations (the pool's
allocation count stays constant).  Here: tq2_gemm never allocates; blr_forward,
blr_forward_paths and blr_backward_paths keep their intermediates in one
grow-only buffer per (device, stream), counted by tq2_workspace_allocs.
"""

import numpy as np
import pytest

import bit_weight_gemm_amd as bw
import workloads as wl
from gpu_util import bits_dev, note, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _blr_dev(d):
    return [bits_dev(d["bits_u"]), bits_dev(d["bits_v"]), to_dev(d["h"]), to_dev(d["l"]), to_dev(d["g"]),
            to_dev(d["x"])]


def test_pool_allocation_count_is_constant_after_warmup(torch):
    stream = torch.cuda.Stream()  # a stream of its own, so earlier tests' pools do not count
    big = wl.blr_inputs()          # M=512, d_in=d_out=4096, r=1024
    big_dev = _blr_dev(big)
    y_big = torch.empty((512, 4096), device="cuda")
    smaller = [wl.blr_inputs(m=m, d_in=di, d_out=do, r=r, index=50 + i)
               for i, (m, di, do, r) in enumerate([(1, 4096, 4096, 1024), (64, 512, 4096, 256), (511, 4096, 4096, 992),
                                                   (7, 96, 40, 32), (200, 1024, 1024, 512), (512, 4096, 128, 1024)])]
    small_dev = [_blr_dev(d) for d in smaller]
    small_y = [torch.empty((d["x"].shape[0], d["h"].size), device="cuda") for d in smaller]
    aos, x_np = wl.prefill_inputs()
    w = bw.tq2_upload(aos, 4096, 4096)
    gemm_ms = (2048, 1, 3, 8, 40, 300, 1024)
    xs = [to_dev(x_np[:m].copy()) for m in gemm_ms]
    ys = [torch.empty((m, 4096), device="cuda") for m in gemm_ms]
    try:
        with torch.cuda.stream(stream):
            before = bw.tq2_workspace_allocs()
            note("[pool] warm-up at the largest size")
            bw.blr_forward(*big_dev, y_big, stream=stream)
            bw.tq2_gemm(w, xs[0], ys[0], stream=stream)
            torch.cuda.synchronize()
            warmed = bw.tq2_workspace_allocs()
            assert warmed == before + 1, "the first call on a stream allocates its workspace once"

            def smaller_calls():
                for i in range(6):
                    bw.blr_forward(*small_dev[i], small_y[i], stream=stream)
                    bw.tq2_gemm(w, xs[1 + i], ys[1 + i], stream=stream)
                torch.cuda.synchronize()

            note("[pool] 12 smaller calls")
            smaller_calls()
            assert bw.tq2_workspace_allocs() == warmed, "smaller calls must not allocate"
            free_before = torch.cuda.mem_get_info()[0]
            smaller_calls()
            assert bw.tq2_workspace_allocs() == warmed
            assert torch.cuda.mem_get_info()[0] == free_before, "device memory grew during smaller calls"
            assert np.isfinite(small_y[3].cpu().numpy()).all()
    finally:
        w.close()


def test_pool_grows_once_for_a_larger_call_and_per_stream(torch):
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    small = wl.blr_inputs(m=16, d_in=256, d_out=128, r=64, index=60)
    large = wl.blr_inputs(m=300, d_in=2048, d_out=512, r=512, index=61)
    sd, ld = _blr_dev(small), _blr_dev(large)
    ys = torch.empty((16, 128), device="cuda")
    yl = torch.empty((300, 512), device="cuda")
    n0 = bw.tq2_workspace_allocs()
    note("[pool] growth and per-stream buffers")
    bw.blr_forward(*sd, ys, stream=s1)
    torch.cuda.synchronize()
    assert bw.tq2_workspace_allocs() == n0 + 1
    bw.blr_forward(*ld, yl, stream=s1)      # needs more: the buffer is replaced once
    torch.cuda.synchronize()
    assert bw.tq2_workspace_allocs() == n0 + 2
    bw.blr_forward(*sd, ys, stream=s1)      # fits: nothing new
    bw.blr_forward(*ld, yl, stream=s1)
    torch.cuda.synchronize()
    assert bw.tq2_workspace_allocs() == n0 + 2
    bw.blr_forward(*sd, ys, stream=s2)      # another stream has a buffer of its own
    torch.cuda.synchronize()
    assert bw.tq2_workspace_allocs() == n0 + 3
    # the results do not depend on which buffer served them
    a = bw.blr_forward(*sd, stream=s1)
    b = bw.blr_forward(*sd, stream=s2)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("m,d_in,d_out,r", [(70, 384, 256, 128), (300, 4096, 256, 512)])
def test_library_and_caller_workspaces_give_the_same_bits(torch, m, d_in, d_out, r):
    # the second size splits the first product's contraction over workgroups
    d = wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=62)
    dev = _blr_dev(d)
    a = bw.blr_forward(*dev)
    b = bw.blr_forward_ws(*dev)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_binding_rejects_mismatched_shapes(torch):
    """The C ABI cannot see buffer sizes; the binding checks every tensor against the
    sizes it derives from x, h and l before calling it."""
    d = wl.blr_inputs(m=8, d_in=64, d_out=96, r=64, index=63)
    bu, bv, h, l, g, x = _blr_dev(d)
    with pytest.raises(ValueError):
        bw.blr_forward(bu, bv, h, l, g[:32], x)                       # g too short
    with pytest.raises(ValueError):
        bw.blr_forward(bu[:50], bv, h, l, g, x)                      # bits_u rows != d_out
    with pytest.raises(ValueError):
        bw.blr_forward(bu, bv, h, l, g, x, torch.empty((8, 95), device="cuda"))   # y too small
    with pytest.raises(ValueError):
        bw.blr_forward_ws(bu, bv, h, l, g, x, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    zeros = [torch.zeros((1, n), device="cuda") for n in (96, 64, 64)]
    with pytest.raises(ValueError):
        bw.blr_backward_paths(bu[None], bv[None], h[None], l[None], g[None], x,
                              torch.zeros((8, 95), device="cuda"), *zeros)         # dy wrong
    torch.cuda.synchronize()
