"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

The shared object must load and export every entry point that include/*.h
declares; argument errors that the contract says are caught on the host must
come back as TQ2_EINVAL before any device is touched.
"""

import ctypes
import glob
import os
import re

import numpy as np
import pytest

import bit_weight_gemm_amd as bw
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bw.LIB_PATH):
        from bit_weight_gemm_amd import build
        build.build()
    return bw.lib()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for must in ("tq2_upload", "tq2_free", "tq2_gemm", "tq2_gemm_path", "tq2_dequant", "blr_forward",
                 "blr_forward_paths", "blr_backward", "blr_backward_paths", "blr_forward_ws", "blr_forward_paths_ws",
                 "blr_backward_ws", "blr_backward_paths_ws", "blr_workspace_size", "blr_backward_workspace_size",
                 "tq2_select_path", "tq2_set_path", "tq2_set_m_small", "tq2_workspace_allocs", "tq2_strerror",
                 "tq2_version", "tq2_weight_info", "blr_saved_size", "blr_forward_paths_save",
                 "blr_backward_paths_saved"):
        assert must in names, must


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in _declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_strerror_and_version(L):
    assert bw.tq2_strerror(0) == "ok"
    assert "invalid" in bw.tq2_strerror(bw.TQ2_EINVAL)
    assert bw.tq2_strerror(12345) == "unknown status"
    assert "gfx950" in bw.tq2_version()


def _upload_status(L, aos, nbytes, n, k):
    out = ctypes.c_void_p()
    buf = None if aos is None else np.ascontiguousarray(aos, np.uint8)
    ptr = None if buf is None else buf.ctypes.data_as(ctypes.c_void_p)
    return L.tq2_upload(ptr, nbytes, n, k, None, ctypes.byref(out)), out


def test_upload_rejects_bad_arguments_on_the_host(L):
    aos, n, k = wl.tiny_weight()
    assert _upload_status(L, None, aos.size, n, k)[0] == bw.TQ2_EINVAL          # null bytes
    assert _upload_status(L, aos, aos.size - 1, n, k)[0] == bw.TQ2_EINVAL       # wrong byte count
    assert _upload_status(L, aos, aos.size, n, 200)[0] == bw.TQ2_EINVAL         # K % 128 != 0
    assert _upload_status(L, aos, aos.size, 0, k)[0] == bw.TQ2_EINVAL           # N < 1
    assert _upload_status(L, aos[:0], 0, 1, 0)[0] == bw.TQ2_EINVAL              # K < 128
    assert L.tq2_upload(aos.ctypes.data_as(ctypes.c_void_p), aos.size, n, k, None, None) == bw.TQ2_EINVAL


def test_upload_row_count_limit(L):
    """Kernels index rows with 32-bit integers: N above 2^31 - 256 (whose padded count
    would not fit) is refused on the host, before the byte count or any device is
    looked at (without the check these calls would reach the device check)."""
    buf = np.zeros(64, np.uint8)
    out = ctypes.c_void_p()
    ptr = buf.ctypes.data_as(ctypes.c_void_p)
    n_max = (1 << 31) - 256
    assert L.tq2_upload(ptr, (n_max + 1) * 34, n_max + 1, 128, None, ctypes.byref(out)) == bw.TQ2_EINVAL
    assert L.tq2_upload(ptr, (1 << 31) * 34, 1 << 31, 128, None, ctypes.byref(out)) == bw.TQ2_EINVAL


def test_set_path_rejects_unknown_paths(L):
    assert L.tq2_set_path(3) == bw.TQ2_EINVAL
    assert L.tq2_set_path(-1) == bw.TQ2_EINVAL
    old = bw.tq2_set_path(bw.TQ2_PATH_MFMA)
    try:
        assert bw.tq2_select_path(1) == bw.TQ2_PATH_MFMA
        assert bw.tq2_set_path(bw.TQ2_PATH_F32) == bw.TQ2_PATH_MFMA
        assert bw.tq2_select_path(4096) == bw.TQ2_PATH_F32
        bw.tq2_set_path(bw.TQ2_PATH_AUTO)
        assert bw.tq2_select_path(1) == bw.TQ2_PATH_F32 and bw.tq2_select_path(4096) == bw.TQ2_PATH_MFMA
    finally:
        bw.tq2_set_path(old)


def test_workspace_counter_starts_at_zero_without_a_device(L):
    assert bw.tq2_workspace_allocs() == 0


def test_workspace_size_rules(L):
    # f16(l.a) [M][r] (the first product's 32 x 64 tiles make one full round: not split)
    assert bw.blr_workspace_size(512, 4096, 4096, 1024) == 512 * 1024 * 2
    assert bw.blr_workspace_size(1, 4096, 4096, 1024) == 1024 * 2   # too few tiles to split d_in
    # then the partial products of a over the chunks of d_in (f32): four chunks at M=128,
    # two at M=256 and M=1024; d_in below 4096: not split
    assert bw.blr_workspace_size(128, 4096, 4096, 1024) == 128 * 1024 * 2 + 4 * 128 * 1024 * 4
    assert bw.blr_workspace_size(256, 4096, 4096, 1024) == 256 * 1024 * 2 + 2 * 256 * 1024 * 4
    assert bw.blr_workspace_size(1024, 4096, 4096, 1024) == 1024 * 1024 * 2 + 2 * 1024 * 1024 * 4
    assert bw.blr_workspace_size(256, 2048, 4096, 1024) == 256 * 1024 * 2
    assert bw.blr_workspace_size(1, 4096, 4096, 1000) == 0     # r % 32 != 0
    assert bw.blr_workspace_size(1, 0, 4096, 1024) == 0        # d_in < 1
    assert bw.blr_workspace_size(-1, 8, 8, 32) == 0            # M < 0
    assert bw.blr_workspace_size(0, 8, 8, 32) > 0              # M == 0 is valid (no-op)


def test_auto_path_threshold(L):
    old = bw.tq2_set_m_small(4)
    try:
        assert bw.tq2_select_path(1) == bw.TQ2_PATH_F32
        assert bw.tq2_select_path(4) == bw.TQ2_PATH_F32
        assert bw.tq2_select_path(5) == bw.TQ2_PATH_MFMA
        bw.tq2_set_m_small(0)
        assert bw.tq2_select_path(1) == bw.TQ2_PATH_MFMA
    finally:
        bw.tq2_set_m_small(old)


def test_blr_forward_rejects_bad_sizes_on_the_host(L):
    # r % 32 != 0 is refused before any pointer or device is looked at
    assert L.blr_forward(None, None, None, None, None, None, None, 4, 8, 8, 33, None) == bw.TQ2_EINVAL
    assert L.blr_forward_ws(None, None, None, None, None, None, None, 4, 8, 8, 33, None, 0, None) == bw.TQ2_EINVAL
    # a layer needs at least one path; bad sizes are refused as for one path
    assert L.blr_forward_paths(0, None, None, None, None, None, None, None, 4, 8, 8, 32, None) == bw.TQ2_EINVAL
    assert L.blr_forward_paths(2, None, None, None, None, None, None, None, 4, 8, 8, 33, None) == bw.TQ2_EINVAL
    # null operands with tokens present are refused on the host, before any allocation
    assert L.blr_forward(None, None, None, None, None, None, None, 4, 8, 8, 32, None) == bw.TQ2_EINVAL
    assert bw.tq2_workspace_allocs() == 0


def test_blr_backward_rejects_bad_arguments_on_the_host(L):
    f = ctypes.c_float
    # gradient scale not a power of two, r % 32 != 0, no paths
    assert L.blr_backward(None, None, None, None, None, None, None, None, None, None, None, 4, 8, 8, 32, f(3.0),
                          None) == bw.TQ2_EINVAL
    assert L.blr_backward(None, None, None, None, None, None, None, None, None, None, None, 4, 8, 8, 33, f(1.0),
                          None) == bw.TQ2_EINVAL
    assert L.blr_backward_paths(0, None, None, None, None, None, None, None, None, None, None, None, 4, 8, 8, 32,
                                f(1.0), None) == bw.TQ2_EINVAL
    assert L.blr_backward_paths_ws(1, None, None, None, None, None, None, None, None, None, None, None, 4, 8, 8, 32,
                                   f(1.0), None, 0, None) == bw.TQ2_EINVAL


def test_saved_size_rules(L):
    """a [M][r] then c [M][d_out] in f32 per path, each part 256-byte aligned."""
    assert bw.blr_saved_size(1, 512, 4096, 4096, 1024) == 512 * 1024 * 4 + 512 * 4096 * 4
    assert bw.blr_saved_size(2, 3, 40, 24, 64) == 2 * (768 + 512)   # a: 768 bytes; c: 288 -> 512 per path
    assert bw.blr_saved_size(0, 3, 40, 24, 64) == 0      # no paths
    assert bw.blr_saved_size(1, 3, 40, 24, 33) == 0      # r % 32 != 0
    assert bw.blr_saved_size(1, 0, 40, 24, 32) > 0       # M == 0 is valid (no-op)


def test_saved_entry_points_reject_bad_arguments_on_the_host(L):
    f = ctypes.c_float
    assert L.blr_forward_paths_save(1, None, None, None, None, None, None, None, 4, 8, 8, 33, None, 0,
                                    None) == bw.TQ2_EINVAL
    assert L.blr_forward_paths_save(0, None, None, None, None, None, None, None, 4, 8, 8, 32, None, 0,
                                    None) == bw.TQ2_EINVAL
    assert L.blr_backward_paths_saved(1, None, None, None, None, None, None, None, None, None, None, None, 4, 8, 8,
                                      32, f(3.0), None, 0, None) == bw.TQ2_EINVAL
    assert L.blr_backward_paths_saved(1, None, None, None, None, None, None, None, None, None, None, None, 4, 8, 8,
                                      32, f(1.0), None, 0, None) == bw.TQ2_EINVAL
    assert bw.tq2_workspace_allocs() == 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message before touching a device."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
