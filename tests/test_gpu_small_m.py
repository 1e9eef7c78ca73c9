"""GPU parity of the MFMA path's small-M kernels with the oracle.

With K a multiple of 1024, up to 32 rows run the 16x16x32 skinny kernel: eight
waves each take one eighth of K, staging their x into LDS step by step (two steps
held, one or two 16-row blocks), each lane one, two or four output columns by N,
each block's sum scaled by d, the waves' partial tiles added in wave order.  Other
K (a multiple of 512, up to 16 rows with M*K <= 32768, or <= 65536 when N <= 8192)
take the 32x32x16 skinny kernel (x staged whole, d folded into the f16 operand).
Other M <= 32 take 32x64 tiles and 33 <= M <= 64
take 64x64 tiles, whose waves split each step's K (four ways; with K/128 a
multiple of 8, each of the four takes two 64-wide slices of a 512-wide step;
two ways when K has few blocks) and add their partial tiles in a fixed order at
the end.  Up to 32 rows, A is read through a buffer resource whose bound
zero-fills the rows past M.  An odd block count takes the 256-column tiles.
Every branch must meet the MFMA bound 4e-3 * sum_k |x*w| of the ternary GEMM
("oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs", correctness test) and give
the same bits on a repeat.
"""

import numpy as np
import pytest

import bit_weight_gemm_amd as bw
import oracle
import workloads as wl
from gpu_util import MFMA_REL, assert_within, check_tq2_sampled, note, run_tq2, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    return torch_cuda()


# K/128 = 32 (multiple of 8: four k groups of two slices), 12 (multiple of 4
# only: four k groups), 6 (even: two k groups), 3 (odd: 256-column tiles).  K=4096
# runs the 16x16x32 skinny kernel up to M=32, K=1536 the 32x32x16 one up to M=16
# (M*K <= 65536 at this N), and the others the tiled kernels.
KS = [4096, 1536, 768, 384]


@pytest.mark.parametrize("k", KS)
@pytest.mark.parametrize("m", [1, 5, 8, 12, 16, 31, 32, 33, 64])
def test_small_m_tiles_match_oracle(torch, m, k):
    n = 1000  # 16 column tiles, the last one partial
    aos = wl.sweep_weight(n, k)
    x = wl.sweep_x(m, k)
    y64, b = oracle.gemm(aos, n, k, x)
    w = bw.tq2_upload(aos, n, k)
    try:
        note(f"[small-M] M={m} N={n} K={k}")
        y = run_tq2(w, x, "mfma")
        assert not np.isnan(y).any()
        assert_within(y, y64, b, MFMA_REL, f"small-M M={m} K={k}")
        again = run_tq2(w, x, "mfma")
        assert np.array_equal(y.view(np.uint32), again.view(np.uint32)), "not deterministic"
    finally:
        w.close()


def test_rows_are_independent(torch):
    """Reversing the rows of x reverses the rows of y bit for bit (no row reads another's A)."""
    n, k, m = 14336, 4096, 8
    aos = wl.sweep_weight(n, k)
    x = wl.sweep_x(m, k)
    w = bw.tq2_upload(aos, n, k)
    try:
        note("[small-M] row reversal M=8 N=14336")
        y = run_tq2(w, x, "mfma")
        yr = run_tq2(w, x[::-1].copy(), "mfma")
        assert np.array_equal(yr.view(np.uint32), y[::-1].view(np.uint32))
        # a single row gives the same bits as that row inside the 8-row call
        y1 = run_tq2(w, x[3:4].copy(), "mfma")
        assert np.array_equal(y1.view(np.uint32), y[3:4].view(np.uint32))
    finally:
        w.close()


@pytest.mark.parametrize("n", [14336, 6000])
def test_every_m_up_to_32_sampled(torch, n):
    """Every row count the skinny kernel takes, M = 1..32, at K = 4096: at the MLP's
    N = 14336 (four columns per lane) and at N = 6000 (two columns per lane), so each
    steps-in-flight, pieces-per-step and row-block configuration and the unrolled
    passes run once; sampled outputs against the oracle."""
    k = 4096
    aos = wl.mlp_inputs(1)[0] if n == 14336 else wl.sweep_weight(n, k)
    x32 = wl.random_x(32, k, 7)
    w = bw.tq2_upload(aos, n, k)
    try:
        for m in range(1, 33):
            check_tq2_sampled(aos, n, k, np.ascontiguousarray(x32[:m]), "mfma", f"every M: M={m} N={n}", count=1024,
                              w=w)
    finally:
        w.close()
