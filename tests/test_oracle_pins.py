"""Pins of the CPU oracle against things other than itself.

Each check is tied to what the pages fix (the block layout and decode of the
ternary-GEMM page's correctness test, the BLR layer's forward equations and bit
mapping on the trainer page) or to mathematics: hand-derived golden values,
exact rational brute force, closed forms, invariants and an independent numpy
evaluation.  A plausible slip in the oracle (wrong slot order, wrong block
offset, dropped scale, sign error, transposed bitmap) fails at least one.
"""

import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U53 = 2.0 ** -53


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _block_bytes(case):
    b = bytearray([int(case["fill"], 16)] * 32)
    for i, v in case["bytes"].items():
        b[int(i)] = int(v, 16)
    d = int(case["d"], 16)
    return bytes(b) + struct.pack("<H", d)


def _expected_block(case):
    w = np.full(128, float(case["expect"]), dtype=np.float32)
    for e, v in case["nonzero"].items():
        w[int(e)] = v
    return w


def _same_bits(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


# ------------------------------------------------------------------ independent decode (pure Python)

def _py_half(bits):
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def _py_weights_exact(aos, n, k):
    """Fractions W[n][k] decoded with Python integer ops and struct's binary16."""
    nb = k // 128
    raw = bytes(np.asarray(aos, np.uint8))
    W = []
    for row in range(n):
        wr = []
        for kb in range(nb):
            off = (row * nb + kb) * 34
            d = Fraction(_py_half(raw[off + 32] | (raw[off + 33] << 8)))
            for e in range(128):
                code = (raw[off + e // 4] >> (2 * (e % 4))) & 3
                wr.append((code - 1) * d)
        W.append(wr)
    return W


def _np_weights(aos, n, k):
    """numpy decode used for larger cross-checks (independent of oracle.c)."""
    blocks = np.asarray(aos, np.uint8).reshape(n, k // 128, 34)
    qs = blocks[:, :, :32]
    codes = np.stack([(qs >> s) & 3 for s in (0, 2, 4, 6)], axis=-1).reshape(n, k // 128, 128)
    d = blocks[:, :, 32:34].copy().view("<f2").astype(np.float64)  # [n][kb][1]
    return ((codes.astype(np.float64) - 1.0) * d).reshape(n, k)


# ------------------------------------------------------------------ f16 and decode

def test_half_decode_matches_struct_for_all_patterns():
    for bits in range(1 << 16):
        got = oracle.half_to_double(bits)
        want = _py_half(bits)
        if np.isnan(want):
            assert np.isnan(got), hex(bits)
        else:
            assert got == want and np.signbit(got) == np.signbit(want), hex(bits)


def test_decode_golden_blocks():
    g = _load("tq2_decode_blocks.json")
    for case in g["cases"]:
        w = oracle.dequant(np.frombuffer(_block_bytes(case), np.uint8), 1, 128)
        assert _same_bits(w[0], _expected_block(case)), case["name"]


def test_decode_golden_composite_addressing():
    g = _load("tq2_decode_blocks.json")
    cases = {c["name"]: c for c in g["cases"]}
    comp = g["composite"]
    n, k = comp["N"], comp["K"]
    raw = b"".join(_block_bytes(cases[name]) for row in comp["blocks"] for name in row)
    w = oracle.dequant(np.frombuffer(raw, np.uint8), n, k)
    for row, names in enumerate(comp["blocks"]):
        for kb, name in enumerate(names):
            assert _same_bits(w[row, kb * 128:(kb + 1) * 128], _expected_block(cases[name])), (row, kb, name)


def test_decode_matches_pure_python_on_tiny_weight():
    aos, n, k = wl.tiny_weight()
    w = oracle.dequant(aos, n, k)
    exact = _py_weights_exact(aos, n, k)
    assert np.array_equal(w.astype(np.float64), np.array([[float(v) for v in r] for r in exact]))


def test_decode_rejects_bad_shapes():
    aos, n, k = wl.tiny_weight()
    with pytest.raises(oracle.OracleError):
        oracle.dequant(aos, n, 200)            # K not a multiple of 128
    with pytest.raises(oracle.OracleError):
        oracle.dequant(aos[:-1], n, k)         # byte count off by one


# ------------------------------------------------------------------ GEMM

def test_gemm_golden_worked_example():
    g = _load("tq2_gemm_worked.json")
    rows = []
    for key in ("row0", "row1"):
        rows.append(_block_bytes(g[key]))
    aos = np.frombuffer(b"".join(rows), np.uint8)
    x = np.stack([np.ones(128, np.float32), np.arange(128, dtype=np.float32)])
    y, b = oracle.gemm(aos, g["N"], g["K"], x)
    assert np.array_equal(y, np.array(g["y"]))
    assert np.array_equal(b, np.array(g["bound"]))


def test_gemm_exact_bruteforce_4x256x40():
    """The 4x256x40 brute-force case: exact rationals vs the f64 oracle."""
    aos, n, k = wl.tiny_weight()
    x = wl.tiny_x(4, k)
    W = _py_weights_exact(aos, n, k)
    y, b = oracle.gemm(aos, n, k, x)
    xf = [[Fraction(float(v)) for v in row] for row in x]
    for m in range(4):
        for j in range(n):
            terms = [xf[m][kk] * W[j][kk] for kk in range(k)]
            exact = sum(terms, Fraction(0))
            babs = sum((abs(t) for t in terms), Fraction(0))
            assert abs(b[m, j] - float(babs)) <= k * U53 * float(babs)
            assert abs(Fraction(y[m, j]) - exact) <= Fraction(k * U53) * babs, (m, j)


def test_gemm_at_matches_exact_values():
    aos, n, k = wl.tiny_weight()
    x = wl.tiny_x(9, k)
    W = _py_weights_exact(aos, n, k)
    rng = np.random.default_rng(5)
    mi = rng.integers(0, 9, 25)
    ni = rng.integers(0, n, 25)
    y, b = oracle.gemm_at(aos, n, k, x, mi, ni)
    for s in range(25):
        terms = [Fraction(float(x[mi[s], kk])) * W[ni[s]][kk] for kk in range(k)]
        exact = sum(terms, Fraction(0))
        babs = sum((abs(t) for t in terms), Fraction(0))
        assert abs(Fraction(y[s]) - exact) <= Fraction(k * U53) * babs


def test_gemm_all_codes_one_gives_exact_zero():
    codes = np.ones((7, 384), np.uint8)
    aos = wl.pack_tq2_aos(codes, wl.f16_bits(np.linspace(0.01, 3, 21).reshape(7, 3)))
    y, b = oracle.gemm(aos, 7, 384, np.random.default_rng(0).standard_normal((5, 384)).astype(np.float32))
    assert np.all(y == 0.0) and np.all(b == 0.0)


@pytest.mark.parametrize("code,sign", [(2, 1.0), (0, -1.0)])
def test_gemm_single_code_gives_plus_minus_d_x(code, sign):
    rng = np.random.default_rng(11 + code)
    n, k = 5, 384
    for _ in range(6):
        codes = np.ones((n, k), np.uint8)
        row, col = int(rng.integers(n)), int(rng.integers(k))
        codes[row, col] = code
        sbits = wl.f16_bits(rng.uniform(0.01, 4.0, (n, k // 128)))
        aos = wl.pack_tq2_aos(codes, sbits)
        x = rng.standard_normal((3, k)).astype(np.float32)
        y, _ = oracle.gemm(aos, n, k, x)
        d = float(sbits.view(np.float16)[row, col // 128])
        want = np.zeros((3, n))
        want[:, row] = sign * d * x[:, col].astype(np.float64)
        assert np.array_equal(y, want)


def test_gemm_all_minus_closed_form():
    rng = np.random.default_rng(3)
    n, k = 4, 512
    sbits = wl.f16_bits(rng.uniform(0.01, 2.0, (n, k // 128)))
    aos = wl.pack_tq2_aos(np.zeros((n, k), np.uint8), sbits)
    x = rng.standard_normal((3, k)).astype(np.float32)
    y, b = oracle.gemm(aos, n, k, x)
    d = sbits.view(np.float16)
    for m in range(3):
        for j in range(n):
            exact = -sum(Fraction(float(d[j, kb])) * sum(Fraction(float(v)) for v in x[m, kb * 128:(kb + 1) * 128])
                         for kb in range(k // 128))
            assert abs(Fraction(y[m, j]) - exact) <= Fraction(k * U53) * Fraction(b[m, j])


def test_gemm_invariants_negation_and_power_of_two_scale():
    rng = np.random.default_rng(21)
    n, k = 9, 640
    codes = rng.integers(0, 3, (n, k)).astype(np.uint8)
    d = rng.uniform(0.01, 1.0, (n, k // 128))
    x = rng.standard_normal((4, k)).astype(np.float32)
    y, _ = oracle.gemm(wl.pack_tq2_aos(codes, wl.f16_bits(d)), n, k, x)
    swapped = np.where(codes == 0, 2, np.where(codes == 2, 0, codes)).astype(np.uint8)
    y_neg, _ = oracle.gemm(wl.pack_tq2_aos(swapped, wl.f16_bits(d)), n, k, x)
    assert np.array_equal(y_neg, -y)
    for j in (-3, 2):
        d2 = wl.f16_bits(d).view(np.float16).astype(np.float64) * 2.0 ** j  # exact in f16 for this range
        y2, _ = oracle.gemm(wl.pack_tq2_aos(codes, wl.f16_bits(d2)), n, k, x)
        assert np.array_equal(y2, y * 2.0 ** j)


def test_gemm_linearity_in_x():
    rng = np.random.default_rng(8)
    n, k = 6, 256
    aos = wl.pack_tq2_aos(rng.integers(0, 3, (n, k)).astype(np.uint8), wl.f16_bits(rng.uniform(0.01, 1, (n, 2))))
    x1 = rng.integers(-50, 50, (3, k)).astype(np.float32)
    x2 = (rng.integers(-50, 50, (3, k)) / 8.0).astype(np.float32)
    y1, b1 = oracle.gemm(aos, n, k, x1)
    y2, b2 = oracle.gemm(aos, n, k, x2)
    y12, _ = oracle.gemm(aos, n, k, (x1 + x2).astype(np.float32))  # x1+x2 is exact in f32
    assert np.all(np.abs(y12 - (y1 + y2)) <= 3 * k * U53 * (b1 + b2))


@pytest.mark.parametrize("n,k", [(8, 128), (40, 256), (8, 3072), (40, 3072)])
def test_gemm_matches_numpy_on_sweep_shapes(n, k):
    aos = wl.sweep_weight(n, k)
    x = wl.sweep_x(33, k)
    y, b = oracle.gemm(aos, n, k, x)
    ref = x.astype(np.float64) @ _np_weights(aos, n, k).T
    assert np.all(np.abs(y - ref) <= 2 * k * U53 * b)


@pytest.mark.parametrize("m", wl.TINY_MS)
def test_page_assertions_on_tiny_workload(m):
    """The page's own check: |GPU - f32 reference| < 1e-3 and output not all zero;
    here the oracle stands in for the GPU against the page's f32 reference."""
    aos, n, k = wl.tiny_weight()
    x = wl.tiny_x(m, k)
    y, b = oracle.gemm(aos, n, k, x)
    y32 = oracle.gemm_f32seq(aos, n, k, x)
    assert np.max(np.abs(y - y32)) < 1e-3
    assert np.any(np.abs(y) > 1e-6)
    # The f32 sequential sum is within its textbook error bound of the exact value.
    assert np.all(np.abs(y32 - y) <= (k * 2.0 ** -24 + k * U53) * b)


# ------------------------------------------------------------------ BLR layer

def _np_signs(bits, r):
    bits = np.asarray(bits, np.uint32)
    by = bits.view(np.uint8).reshape(bits.shape[0], -1)
    s = np.unpackbits(by, axis=1, bitorder="little")[:, :r]
    return np.where(s == 1, 1.0, -1.0)


def _np_blr(d):
    r = d["l"].size
    sv = _np_signs(d["bits_v"], r)
    su = _np_signs(d["bits_u"], r)
    x = d["x"].astype(np.float64)
    a = (x * d["g"].astype(np.float64)) @ sv
    c = (a * d["l"].astype(np.float64)) @ su.T
    return c * d["h"].astype(np.float64), a, su, sv


def _triple_abs(d):
    """|h_i| * sum_k l_k * sum_j |x_j g_j| per output: a bound on every partial sum."""
    s = np.abs(d["x"].astype(np.float64) * d["g"].astype(np.float64)).sum(axis=1)
    return np.abs(d["h"].astype(np.float64))[None, :] * s[:, None] * np.abs(d["l"].astype(np.float64)).sum()


def test_blr_golden_worked_example():
    g = _load("blr_worked.json")
    d = dict(bits_u=np.array(g["bits_u"], np.uint32)[:, None], bits_v=np.array(g["bits_v"], np.uint32)[:, None],
             h=np.array(g["h"], np.float32), l=np.array(g["l"], np.float32), g=np.array(g["g"], np.float32),
             x=np.array(g["x"], np.float32))
    y, a = oracle.blr_forward(**d, want_a=True)
    assert np.array_equal(y, np.array(g["y"])) and np.array_equal(a, np.array(g["a"]))
    b = oracle.blr_bound_at(**d, ti=[0, 0], ii=[0, 1])
    assert np.array_equal(b, np.array(g["bound"][0]))


@pytest.mark.parametrize("fill", [0xFFFFFFFF, 0])
def test_blr_uniform_signs_closed_form(fill):
    """All signs equal: S_U S_V^T entries are all +1, so y = h_i (sum_k l_k)(sum_j g_j x_j)."""
    d = wl.blr_inputs(m=3, d_in=40, d_out=24, r=64, index=7)
    d["bits_u"][:] = fill
    d["bits_v"][:] = fill
    y, _ = oracle.blr_forward(**d)
    sl = sum(Fraction(float(v)) for v in d["l"])
    for t in range(3):
        sx = sum(Fraction(float(d["g"][j])) * Fraction(float(d["x"][t, j])) for j in range(40))
        for i in range(24):
            exact = Fraction(float(d["h"][i])) * sl * sx
            tri = float(abs(Fraction(float(d["h"][i]))) * sl * sum(abs(Fraction(float(d["g"][j]) * float(d["x"][t, j]))) for j in range(40)))
            assert abs(Fraction(y[t, i]) - exact) <= Fraction((40 + 64 + 3) * U53 * tri)


def test_blr_dense_equivalence_exact():
    """y = x W^T with W^ = diag(h) S_U diag(l) S_V^T diag(g), all in exact rationals."""
    m, d_in, d_out, r = 3, 40, 24, 64
    d = wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=9)
    y, _ = oracle.blr_forward(**d)
    su = _np_signs(d["bits_u"], r)
    sv = _np_signs(d["bits_v"], r)
    F = lambda v: Fraction(float(v))
    l = [F(v) for v in d["l"]]
    W = [[F(d["h"][i]) * F(d["g"][j]) * sum((int(su[i, k]) * l[k] * int(sv[j, k]) for k in range(r)), Fraction(0))
          for j in range(d_in)] for i in range(d_out)]
    tri = _triple_abs(d)
    for t in range(m):
        for i in range(d_out):
            exact = sum((F(d["x"][t, j]) * W[i][j] for j in range(d_in)), Fraction(0))
            assert abs(Fraction(y[t, i]) - exact) <= Fraction((d_in + r + 3) * U53 * tri[t, i]), (t, i)
    # the dense-equivalent bound of a few outputs, exactly
    ti, ii = np.array([0, 1, 2, 2]), np.array([0, 5, 17, 23])
    b = oracle.blr_bound_at(**d, ti=ti, ii=ii)
    for s in range(4):
        t, i = ti[s], ii[s]
        exact = sum((abs(F(d["x"][t, j]) * W[i][j]) for j in range(d_in)), Fraction(0))
        assert abs(Fraction(b[s]) - exact) <= Fraction(2 * (d_in + r) * U53) * exact


def test_blr_flip_identities_pin_bit_mapping():
    """Flipping S_U[i][k] changes only column i, by -2 S_U[i][k] h_i l_k a[t][k];
    flipping S_V[j][k] changes y[t][i] by -2 S_V[j][k] g_j x[t][j] l_k h_i S_U[i][k]."""
    m, d_in, d_out, r = 5, 48, 40, 96
    d = wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=11)
    y0, a = oracle.blr_forward(**d, want_a=True)
    _, a_np, su, sv = _np_blr(d)
    assert np.allclose(a, a_np, rtol=0, atol=1e-12 * np.abs(a_np).max())
    tri = _triple_abs(d)
    h, l, g, x = (d[k].astype(np.float64) for k in ("h", "l", "g", "x"))
    for (i, k) in [(0, 0), (3, 31), (39, 32), (17, 95), (20, 64)]:
        e = dict(d)
        e["bits_u"] = d["bits_u"].copy()
        e["bits_u"][i, k // 32] ^= np.uint32(1 << (k % 32))
        y1, _ = oracle.blr_forward(**e)
        want = np.zeros_like(y0)
        want[:, i] = -2.0 * su[i, k] * h[i] * l[k] * a_np[:, k]
        assert np.all(np.abs((y1 - y0) - want) <= 4 * (d_in + r + 3) * U53 * tri)
    for (j, k) in [(0, 0), (47, 31), (5, 32), (30, 95)]:
        e = dict(d)
        e["bits_v"] = d["bits_v"].copy()
        e["bits_v"][j, k // 32] ^= np.uint32(1 << (k % 32))
        y1, _ = oracle.blr_forward(**e)
        want = -2.0 * sv[j, k] * g[j] * x[:, j][:, None] * l[k] * (h * su[:, k])[None, :]
        assert np.all(np.abs((y1 - y0) - want) <= 4 * (d_in + r + 3) * U53 * tri)


def test_blr_matches_numpy_on_trainer_test_shapes():
    """The trainer test's shapes (m=256 outputs, n=384 inputs, r=128, 70 tokens): oracle vs numpy f64."""
    d = wl.blr_page_inputs()
    y, _ = oracle.blr_forward(**d)
    ref, _, _, _ = _np_blr(d)
    assert np.all(np.abs(y - ref) <= 2 * (384 + 128 + 3) * U53 * _triple_abs(d))


def test_blr_rejects_bad_arguments():
    d = wl.blr_inputs(m=2, d_in=8, d_out=8, r=32, index=1)
    with pytest.raises(oracle.OracleError):
        oracle.blr_bound_at(**d, ti=[2], ii=[0])   # token index out of range


def test_blr_paths_cancel_and_add_exactly():
    """A layer is the sum of its paths: a second path equal to the first but with every
    S_U sign flipped gives c_1 = -c_0 exactly, so the layer output is exactly zero;
    two equal paths give exactly twice one path (scaling by 2 is exact in f64)."""
    d = wl.blr_inputs(m=5, d_in=40, d_out=24, r=64, index=11)
    x = d.pop("x")
    flipped = dict(d, bits_u=~d["bits_u"])
    assert np.all(oracle.blr_forward_paths([d, flipped], x) == 0.0)
    one, _ = oracle.blr_forward(**d, x=x)
    assert np.array_equal(oracle.blr_forward_paths([d, d], x), 2.0 * one)
    assert np.array_equal(oracle.blr_forward_paths([d], x), one)


def test_blr_paths_dense_equivalence_exact():
    """Two different paths against y = x (W^_0 + W^_1)^T in exact rationals: each path
    within its own f64 error bound (as for one path), plus one rounding of the sum."""
    m, d_in, d_out, r = 2, 24, 16, 32
    paths = [wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=12 + p) for p in range(2)]
    x = paths[0]["x"]
    for d in paths:
        d["x"] = x
    y = oracle.blr_forward_paths(paths, x)
    F = lambda v: Fraction(float(v))
    W = [[Fraction(0)] * d_in for _ in range(d_out)]
    tri = np.zeros((m, d_out))
    for d in paths:
        su, sv = _np_signs(d["bits_u"], r), _np_signs(d["bits_v"], r)
        l = [F(v) for v in d["l"]]
        for i in range(d_out):
            for j in range(d_in):
                W[i][j] += F(d["h"][i]) * F(d["g"][j]) * sum((int(su[i, k]) * l[k] * int(sv[j, k]) for k in range(r)), Fraction(0))
        tri += _triple_abs(d)
    for t in range(m):
        for i in range(d_out):
            exact = sum((F(x[t, j]) * W[i][j] for j in range(d_in)), Fraction(0))
            err = abs(Fraction(y[t, i]) - exact)
            assert err <= Fraction((d_in + r + 3) * U53 * tri[t, i]) + Fraction(U53) * abs(Fraction(y[t, i])), (t, i)


def test_blr_backward_euler_identities():
    """The layer is linear in each of x, h, l and g, so with s = sum dy.y (y from the
    forward oracle, a separate implementation) the backward must satisfy
    s = sum x.dx = sum_i h_i dh_i = sum_k l_k dl_k = sum_j g_j dg_j (per path for h, l,
    g; one path here).  A dropped factor, a transposed sign matrix or a wrong operand in
    any gradient breaks one of the four."""
    d = wl.blr_inputs(m=7, d_in=40, d_out=24, r=64, index=13)
    x = d.pop("x")
    dy = np.random.default_rng(5).standard_normal((7, 24)).astype(np.float32)
    y, _ = oracle.blr_forward(**d, x=x)
    s = float(np.sum(dy.astype(np.float64) * y))
    dx, [(dh, dl, dg)] = oracle.blr_backward_paths([d], x, dy)
    scale = float(np.sum(np.abs(dy.astype(np.float64) * y))) + abs(s)
    for other in (np.sum(x.astype(np.float64) * dx), np.sum(d["h"].astype(np.float64) * dh),
                  np.sum(d["l"].astype(np.float64) * dl), np.sum(d["g"].astype(np.float64) * dg)):
        assert abs(other - s) <= 1e-12 * scale


def test_blr_backward_dx_is_the_transposed_product_exactly():
    """dx = dy W^ with W^ = diag(h) S_U diag(l) S_V^T diag(g), summed over two paths, in
    exact rationals on a tiny layer."""
    m, d_in, d_out, r = 2, 12, 8, 32
    paths = [wl.blr_inputs(m=m, d_in=d_in, d_out=d_out, r=r, index=15 + p) for p in range(2)]
    x = paths[0]["x"]
    dy = (np.arange(m * d_out, dtype=np.float32).reshape(m, d_out) * np.float32(0.125) - np.float32(0.9))
    dx, _ = oracle.blr_backward_paths(paths, x, dy)
    F = lambda v: Fraction(float(v))
    for t in range(m):
        for j in range(d_in):
            exact = Fraction(0)
            for d in paths:
                su, sv = _np_signs(d["bits_u"], r), _np_signs(d["bits_v"], r)
                for i in range(d_out):
                    w = F(d["h"][i]) * F(d["g"][j]) * sum((int(su[i, k]) * F(d["l"][k]) * int(sv[j, k]) for k in range(r)), Fraction(0))
                    exact += F(dy[t, i]) * w
            assert abs(Fraction(dx[t, j]) - exact) <= Fraction(1, 10**9) * (abs(exact) + 1)
