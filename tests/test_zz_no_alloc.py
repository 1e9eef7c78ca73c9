"""blr_forward_noalloc: the binary low-rank forward with its workspace in the
library's static device scratch, for callers that cannot allocate.

It must give blr_forward's bits (same kernels), on two calls in a row with the
second one smaller (the scratch keeps the first call's contents), allocate
nothing (no library workspace, no device memory), and refuse sizes beyond its
scratch before queueing anything.  Called through the C ABI.
"""

import ctypes

import numpy as np
import pytest

import bit_weight_gemm_amd as bw
import workloads as wl
from gpu_util import bits_dev, note, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


def _noalloc(torch, d, stream, check_memory):
    m, d_in = d["x"].shape
    d_out, r = d["h"].size, d["l"].size
    ops = [bits_dev(d["bits_u"]), bits_dev(d["bits_v"]), to_dev(d["h"]), to_dev(d["l"]), to_dev(d["g"]),
           to_dev(d["x"])]
    base = torch.full((m * d_out + 64,), float("nan"), device="cuda")
    y = base[: m * d_out].view(m, d_out)
    torch.cuda.synchronize()
    allocs, free = bw.tq2_workspace_allocs(), torch.cuda.mem_get_info()[0]
    st = bw.lib().blr_forward_noalloc(*[ctypes.c_void_p(t.data_ptr()) for t in ops], ctypes.c_void_p(y.data_ptr()),
                                      m, d_in, d_out, r, ctypes.c_void_p(stream.cuda_stream))
    assert st == bw.TQ2_OK, bw.tq2_strerror(st)
    torch.cuda.synchronize()
    assert bw.tq2_workspace_allocs() == allocs, "blr_forward_noalloc allocated a workspace"
    if check_memory:  # after the first call on the device, which looks up (and may load) the static array
        assert torch.cuda.mem_get_info()[0] == free, "device memory changed during blr_forward_noalloc"
    assert np.isnan(base[m * d_out:].cpu().numpy()).all(), "write past the end of y"
    out = y.cpu().numpy()
    assert not np.isnan(out).any(), "unwritten outputs"
    return out, ops


def test_noalloc_matches_blr_forward_on_two_calls(torch):
    stream = torch.cuda.Stream()
    cases = [wl.blr_inputs(), wl.blr_inputs(m=70, d_in=384, d_out=256, r=128, index=71)]  # second one smaller
    outs = []
    for i, d in enumerate(cases):
        note(f"[noalloc] M={d['x'].shape[0]} d_in={d['x'].shape[1]} d_out={d['h'].size} r={d['l'].size}")
        y, ops = _noalloc(torch, d, stream, check_memory=i > 0)
        outs.append((y, ops))
    again, _ = _noalloc(torch, cases[0], stream, check_memory=True)
    assert np.array_equal(again.view(np.uint32), outs[0][0].view(np.uint32))
    for (y, ops) in outs:
        want = bw.blr_forward(*ops, stream=stream)
        torch.cuda.synchronize()
        assert np.array_equal(y.view(np.uint32), want.cpu().numpy().view(np.uint32))


def test_noalloc_refuses_sizes_beyond_its_scratch(torch):
    m, d_in, d_out, r = 16384, 4096, 4096, 1024
    assert bw.blr_workspace_size(m, d_in, d_out, r) > bw.TQ2_STATIC_SCRATCH_BYTES
    # refused from the sizes alone, before any pointer or device is looked at
    st = bw.lib().blr_forward_noalloc(None, None, None, None, None, None, None, m, d_in, d_out, r, None)
    assert st == bw.TQ2_ETOOBIG
    assert "static" in bw.tq2_strerror(st)
