"""The library's calls inside a captured HIP graph.

Callers that capture their work in graphs (the bench does, and so do serving
loops) need every call to be capturable once warmed up: no allocation, no
host synchronisation and no memset node.  A graph holding ternary GEMMs on
both paths, a binary low-rank forward on the library's workspace (at a size
whose first product is one launch, and at one whose contraction is split over
workgroups with a launch that adds the chunks), one on the fixed scratch
(blr_forward_noalloc) and the backward from saved activations is
replayed several times (with the ternary GEMM also at M=8 and M=24, the skinny
kernel with one and two row blocks), with other eager library work and synchronisations in
between, and every replay must give the eager results bit for bit; after the
inputs are overwritten in place, a replay must give the eager results on the
new inputs.
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


def test_graph_replays_match_eager(torch):
    note("[graph] capture of tq2_gemm (both paths), blr_forward, blr_forward_noalloc, both backwards")
    aos, n, k = wl.random_weight(1000, 1024, 31), 1000, 1024
    w = bw.tq2_upload(aos, n, k)
    x1 = to_dev(wl.random_x(1, k, 32))
    x100 = to_dev(wl.random_x(100, k, 33))
    x8, x24 = to_dev(wl.random_x(8, k, 41)), to_dev(wl.random_x(24, k, 42))
    d = wl.blr_inputs(m=70, d_in=384, d_out=256, r=128, index=34)
    bu, bv = bits_dev(d["bits_u"]), bits_dev(d["bits_v"])
    h, l, g, xb = to_dev(d["h"]), to_dev(d["l"]), to_dev(d["g"]), to_dev(d["x"])
    dy = to_dev((np.random.default_rng(35).standard_normal((70, 256)) * 1e-3).astype(np.float32))
    y1, y100 = torch.empty((1, n), device="cuda"), torch.empty((100, n), device="cuda")
    y8, y24 = torch.empty((8, n), device="cuda"), torch.empty((24, n), device="cuda")
    yb, yn = torch.empty((70, 256), device="cuda"), torch.empty((70, 256), device="cuda")
    ys = torch.empty((70, 256), device="cuda")
    saved = torch.empty(bw.blr_saved_size(1, 70, 384, 256, 128), dtype=torch.uint8, device="cuda")
    grads = [torch.zeros((1, m), device="cuda") for m in (256, 128, 384)]
    grads_r = [torch.zeros((1, m), device="cuda") for m in (256, 128, 384)]
    dx, dx_r = torch.empty((70, 384), device="cuda"), torch.empty((70, 384), device="cuda")
    P = lambda t: t[None]  # noqa: E731  (one path)
    # first product split four ways over d_in (10 x 4 tiles of 32 x 128)
    d2 = wl.blr_inputs(m=300, d_in=4096, d_out=256, r=512, index=39)
    b2 = [bits_dev(d2["bits_u"]), bits_dev(d2["bits_v"])] + [to_dev(d2[key]) for key in ("h", "l", "g", "x")]
    y2 = torch.empty((300, 256), device="cuda")

    def work(s):
        bw.tq2_gemm_path(w, x1, y1, bw.TQ2_PATH_F32, stream=s)
        bw.tq2_gemm_path(w, x100, y100, bw.TQ2_PATH_MFMA, stream=s)
        bw.tq2_gemm_path(w, x8, y8, bw.TQ2_PATH_MFMA, stream=s)
        bw.tq2_gemm_path(w, x24, y24, bw.TQ2_PATH_MFMA, stream=s)
        bw.blr_forward(bu, bv, h, l, g, xb, yb, stream=s)
        bw.blr_forward(*b2, y2, stream=s)
        bw._check(bw.lib().blr_forward_noalloc(
            bw._dev(bu, torch.int32, "bu"), bw._dev(bv, torch.int32, "bv"), bw._dev(h, torch.float32, "h"),
            bw._dev(l, torch.float32, "l"), bw._dev(g, torch.float32, "g"), bw._dev(xb, torch.float32, "x"),
            bw._dev(yn, torch.float32, "y"), 70, 384, 256, 128, bw._stream(s)), "blr_forward_noalloc")
        bw.blr_forward_paths_save(P(bu), P(bv), P(h), P(l), P(g), xb, ys, saved, stream=s)
        bw.blr_backward_paths_saved(P(bu), P(bv), P(h), P(l), P(g), xb, dy, *grads, saved, dx=dx, stream=s)
        bw.blr_backward_paths(P(bu), P(bv), P(h), P(l), P(g), xb, dy, *grads_r, dx=dx_r, stream=s)

    outs = (y1, y100, yb, yn, ys, dx, y2, y8, y24, dx_r)
    accum = grads + grads_r  # accumulated in place: cleared before each run

    def eager():
        for t in accum:
            t.zero_()
        s = torch.cuda.current_stream()
        work(s)
        torch.cuda.synchronize()
        return [o.cpu().numpy().copy() for o in outs] + [t.cpu().numpy().copy() for t in accum]

    want = eager()                        # warms the library's workspaces up
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(side)                        # the side stream's own workspace, grown before capture
    torch.cuda.synchronize()
    allocs = bw.tq2_workspace_allocs()
    graph = torch.cuda.CUDAGraph()
    for t in accum:
        t.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        work(side)
    assert bw.tq2_workspace_allocs() == allocs   # nothing allocated while capturing

    def replay():
        for t in accum:
            t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            graph.replay()
        torch.cuda.synchronize()
        return [o.cpu().numpy().copy() for o in outs] + [t.cpu().numpy().copy() for t in accum]

    for rep in range(4):
        got = replay()
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (rep, i)
        bw.tq2_gemm_path(w, x100, torch.empty((100, n), device="cuda"), bw.TQ2_PATH_MFMA)  # eager work between
        torch.cuda.synchronize()
    # new inputs in place: the replay must follow them
    x1.copy_(to_dev(wl.random_x(1, k, 36)))
    x100.copy_(to_dev(wl.random_x(100, k, 37)))
    x8.copy_(to_dev(wl.random_x(8, k, 43)))
    xb.copy_(to_dev(wl.random_x(70, 384, 38)))
    b2[5].copy_(to_dev(wl.random_x(300, 4096, 40)))
    torch.cuda.synchronize()
    got = replay()
    want2 = eager()
    for i, (a, b) in enumerate(zip(got, want2)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), ("new inputs", i)
    assert not np.array_equal(want2[0], want[0])
    assert bw.tq2_workspace_allocs() == allocs
    del graph
    w.close()
