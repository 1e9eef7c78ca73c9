"""Seeded synthetic inputs for the TQ2_0_g128 GEMM and the binary low-rank (BLR) layer.

This module only *makes inputs*: weight blocks in the page's array-of-structs byte
layout, activations, sign bitmaps and the per-channel BLR vectors.  It holds none of
the arithmetic being checked (no decode, no products, no sums), so both the CPU
oracle and the HIP path can take their inputs from here without sharing any of
the method.

Sources of the recipes (the pages, cited by title and section):

* "oxibonsai-kernels 0.2.1 -- tests_gemm_tq2.rs", correctness test
  (`test_encode_gemm_tq2_matches_reference`): the tiny N=40, K=256 weight from a
  32-bit LCG with the Numerical Recipes constants, seed 0x12345678, code =
  (state >> 16) % 3, four codes per byte with the first in the low two bits, a
  per-block f16 scale 0.0625 + 0.0078125*(row + 0.5*blk), and the index-derived
  input 0.013*k - 0.4 + 0.0007*m.
* the same page, tiled/simdgroup parity sweeps: seed 0x9E3779B1 ^ (N<<8) ^ K
  (v8) or 0x2545F491 ^ (N<<8) ^ K (v9/v10), scale 0.05 + 0.003*(row % 17) +
  0.002*blk and input sin(0.011*k - 0.37) + 0.0005*m.
* the same page, DiT benchmarks: seed 0xDEADBEEF ^ N, constant scale 0.0625,
  input (i % 251)*0.001 - 0.12.
* "cortiq-engine 0.8.43 -- train_mm.rs", test module: the xorshift generator
  `rnd`, signs taken as +1 where the draw is >= 0, and the bitmap packing (bit j
  of word w is rank index 32w+j, 1 meaning +1).

The larger workloads (decode GEMV, small-batch MLP, prefill, BLR layer) state
only distributions; they are drawn with numpy's PCG64 `default_rng`, seeds
1000+i (weights / bitmaps), 2000+i (activations) and 3000+i (h, l, g) for
workload index i.
"""

from __future__ import annotations

import numpy as np

BLOCK = 128          # weights per TQ2_0_g128 block
BLOCK_BYTES = 34     # 32 code bytes + one little-endian f16 scale

LCG_MUL = 1664525
LCG_ADD = 1013904223


# ----------------------------------------------------------------------------- LCG codes

def lcg_codes(seed: int, count: int) -> np.ndarray:
    """`count` codes in {0,1,2} from the page's LCG, state updated before each draw.

    state <- state*1664525 + 1013904223 (mod 2^32); code = (state >> 16) % 3.
    Evaluated in blocks with the closed-form jump (a^j, c*(a^j-1)/(a-1)) so large
    weights are cheap; the sequence is the same as the one-step recurrence.
    """
    out = np.empty(count, dtype=np.uint8)
    if count == 0:
        return out
    step = min(count, 1 << 14)
    mul = np.empty(step, dtype=np.uint64)
    add = np.empty(step, dtype=np.uint64)
    m, a = 1, 0
    for j in range(step):  # state_{s+j+1} = mul[j]*state_s + add[j]
        m = (m * LCG_MUL) & 0xFFFFFFFF
        a = (a * LCG_MUL + LCG_ADD) & 0xFFFFFFFF
        mul[j] = m
        add[j] = a
    s = np.uint64(seed & 0xFFFFFFFF)
    mask = np.uint64(0xFFFFFFFF)
    done = 0
    while done < count:
        n = min(step, count - done)
        states = (mul[:n] * s + add[:n]) & mask
        out[done:done + n] = ((states >> np.uint64(16)) % np.uint64(3)).astype(np.uint8)
        s = states[n - 1]
        done += n
    return out


def lcg_codes_reference(seed: int, count: int) -> np.ndarray:
    """One-step form of `lcg_codes` (for cross-checking the blocked form)."""
    s = seed & 0xFFFFFFFF
    out = np.empty(count, dtype=np.uint8)
    for i in range(count):
        s = (s * LCG_MUL + LCG_ADD) & 0xFFFFFFFF
        out[i] = (s >> 16) % 3
    return out


# ----------------------------------------------------------------------------- block packing

def f16_bits(values) -> np.ndarray:
    """IEEE binary16 bit patterns of `values`, rounded to nearest-even by numpy."""
    return np.asarray(values).astype(np.float16).view(np.uint16)


def pack_tq2_aos(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Array-of-structs TQ2_0_g128 bytes from codes [N][K] (0..3) and scale bits [N][K/128].

    Block (n, kb) occupies bytes [(n*(K/128)+kb)*34, +34): byte b of the block holds
    elements 4b..4b+3 of the block, element 4b+j in bits 2j..2j+1; bytes 32..33 are
    the f16 scale, little-endian.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 128")
    kb = k // BLOCK
    scale_bits = np.asarray(scale_bits, dtype=np.uint16).reshape(n, kb)
    c = codes.reshape(n, kb, 32, 4).astype(np.uint8)
    qs = (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)
    out = np.empty((n, kb, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, :32] = qs
    out[:, :, 32:34] = scale_bits.astype("<u2").view(np.uint8).reshape(n, kb, 2)
    return out.reshape(-1)


# ----------------------------------------------------------------------------- page workloads

def tiny_weight():
    """N=40, K=256 weight of the page's correctness test: (aos bytes, N, K)."""
    n, k = 40, 256
    codes = lcg_codes(0x12345678, n * k).reshape(n, k)
    row = np.arange(n, dtype=np.float32)[:, None]
    blk = np.arange(k // BLOCK, dtype=np.float32)[None, :]
    scale = np.float32(0.0625) + np.float32(0.0078125) * (row + np.float32(0.5) * blk)
    return pack_tq2_aos(codes, f16_bits(scale.astype(np.float32))), n, k


def tiny_x(m: int, k: int = 256) -> np.ndarray:
    """x[m][k] = (k*0.013 - 0.4) + m*0.0007, each step in f32 (no fused multiply-add)."""
    col = np.arange(k, dtype=np.float32)[None, :]
    row = np.arange(m, dtype=np.float32)[:, None]
    return ((col * np.float32(0.013) - np.float32(0.4)) + row * np.float32(0.0007)).astype(np.float32)


TINY_MS = (1, 7, 8, 9, 100)
SWEEP_MS = (1, 7, 8, 9, 32, 33, 100, 1536)
SWEEP_NS = (8, 40, 3072)
SWEEP_KS = (128, 256, 3072)


def sweep_weight(n: int, k: int, seed_base: int = 0x9E3779B1):
    """Weight of the page's parity sweeps: LCG seeded seed_base ^ (N<<8) ^ K."""
    seed = (seed_base ^ ((n << 8) & 0xFFFFFFFF) ^ k) & 0xFFFFFFFF
    codes = lcg_codes(seed, n * k).reshape(n, k)
    row = (np.arange(n) % 17).astype(np.float32)[:, None]
    blk = np.arange(k // BLOCK, dtype=np.float32)[None, :]
    scale = (np.float32(0.05) + np.float32(0.003) * row) + np.float32(0.002) * blk
    return pack_tq2_aos(codes, f16_bits(scale.astype(np.float32)))


def sweep_x(m: int, k: int) -> np.ndarray:
    """x[m][k] = sin(0.011*k - 0.37) + 0.0005*m in f32."""
    col = np.arange(k, dtype=np.float32)[None, :]
    row = np.arange(m, dtype=np.float32)[:, None]
    t = (col * np.float32(0.011) - np.float32(0.37)).astype(np.float32)
    return (np.sin(t).astype(np.float32) + row * np.float32(0.0005)).astype(np.float32)


DIT_SHAPES = ((1536, 27648, 3072), (1536, 3072, 3072))  # (M, N, K) of the page's DiT benchmarks


def dit_weight(n: int, k: int):
    """Weight of the page's DiT benchmarks: LCG seed 0xDEADBEEF ^ N, scale 0.0625."""
    codes = lcg_codes((0xDEADBEEF ^ n) & 0xFFFFFFFF, n * k).reshape(n, k)
    return pack_tq2_aos(codes, np.full((n, k // BLOCK), f16_bits(np.float32(0.0625)), np.uint16))


def dit_x(m: int, k: int) -> np.ndarray:
    i = np.arange(m * k, dtype=np.int64) % 251
    return (i.astype(np.float32) * np.float32(0.001) - np.float32(0.12)).reshape(m, k).astype(np.float32)


# ----------------------------------------------------------------------------- edge cases of the format

EDGE_CLASSES = 8  # row n of an edge weight belongs to class n % 8


def edge_weight(n: int, k: int, seed: int):
    """A weight exercising the block format's edge cases, row by row.

    Row n has class n % 8:
      0  every code 1 (byte 0x55): the weight is zero whatever the scale;
      1  every code 1 except one code 0 or 2 at a random position;
      2  every code 0 (byte 0x00): every weight is -d;
      3  codes 0..3, every scale an f16 subnormal of either sign;
      4  codes 0..3, every scale with 16384 <= |d| <= 32752 (2d still finite in f16), either sign;
      5  codes 0..3, every scale negative (normal range);
      6  codes 2 and 3 only;
      7  codes 0..3, each block's scale drawn from {+-0, subnormal, normal, large}.
    Other rows' scales are normal f16 values of either sign with |d| <= 32752.
    Returns (aos bytes, codes [n][k] u8, scale bits [n][k/128] u16).
    """
    rng = np.random.default_rng(seed)
    kb = k // BLOCK
    codes = rng.integers(0, 4, (n, k), dtype=np.uint8)
    sign = (rng.integers(0, 2, (n, kb)).astype(np.uint16) << np.uint16(15)).astype(np.uint16)
    normal = rng.integers(0x0400, 0x7800, (n, kb)).astype(np.uint16)     # exponents 1..29: |d| <= 32752
    subnormal = rng.integers(1, 0x0400, (n, kb)).astype(np.uint16)
    large = rng.integers(0x7400, 0x7800, (n, kb)).astype(np.uint16)      # 16384 <= |d| <= 32752
    cls = np.arange(n) % EDGE_CLASSES
    bits = normal.copy()
    codes[cls == 0] = 1
    r1 = np.flatnonzero(cls == 1)
    codes[r1] = 1
    codes[r1, rng.integers(0, k, r1.size)] = rng.choice(np.array([0, 2], np.uint8), r1.size)
    codes[cls == 2] = 0
    bits[cls == 3] = subnormal[cls == 3]
    bits[cls == 4] = large[cls == 4]
    sign[cls == 5] = 0x8000
    r6 = cls == 6
    codes[r6] = rng.integers(2, 4, (int(r6.sum()), k), dtype=np.uint8)
    kind = rng.integers(0, 4, (n, kb))
    mixed = np.where(kind == 0, np.uint16(0), np.where(kind == 1, subnormal, np.where(kind == 2, normal, large)))
    bits[cls == 7] = mixed[cls == 7]
    bits = (bits | sign).astype(np.uint16)
    return pack_tq2_aos(codes, bits), codes, bits


# Seeded distribution workloads (index i: 1 decode, 2 MLP, 3 prefill, 4 BLR).
DECODE = dict(name="decode_gemv", M=1, N=4096, K=4096, index=1)
MLP = dict(name="mlp_up", Ms=(8, 32), N=14336, K=4096, index=2)
PREFILL = dict(name="prefill", M=2048, N=4096, K=4096, index=3)
BLR = dict(name="blr_forward", M=512, d_in=4096, d_out=4096, r=1024, index=4)


def random_weight(n: int, k: int, index: int, probs=None):
    """Codes iid over {0,1,2} (uniform, or with `probs`), scales f16(U(0.01, 0.1))."""
    rng = np.random.default_rng(1000 + index)
    if probs is None:
        codes = rng.integers(0, 3, size=(n, k), dtype=np.uint8)
    else:
        codes = rng.choice(np.array([0, 1, 2], dtype=np.uint8), size=(n, k), p=probs)
    scale = rng.uniform(0.01, 0.1, size=(n, k // BLOCK))
    return pack_tq2_aos(codes, f16_bits(scale))


def random_x(m: int, k: int, index: int, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(2000 + index)
    return (rng.standard_normal((m, k)) * sigma).astype(np.float32)


def decode_inputs():
    c = DECODE
    return random_weight(c["N"], c["K"], 1), random_x(c["M"], c["K"], 1)


def mlp_inputs(m: int):
    c = MLP
    return random_weight(c["N"], c["K"], 2), random_x(m, c["K"], 2)


def prefill_inputs():
    c = PREFILL
    w = random_weight(c["N"], c["K"], 3, probs=[0.25, 0.5, 0.25])
    return w, random_x(c["M"], c["K"], 3, sigma=float(np.sqrt(0.5)))


def blr_inputs(m=None, d_in=None, d_out=None, r=None, index=4):
    """Bitmaps uniform u32, h/l/g f32 U(0.5, 1.5), x f32 N(0, 1).

    Returns dict(bits_u [d_out][r/32] u32, bits_v [d_in][r/32] u32, h [d_out], l [r],
    g [d_in], x [m][d_in]).
    """
    c = BLR
    m = c["M"] if m is None else m
    d_in = c["d_in"] if d_in is None else d_in
    d_out = c["d_out"] if d_out is None else d_out
    r = c["r"] if r is None else r
    words = (r + 31) // 32
    rb = np.random.default_rng(1000 + index)
    bits_u = rb.integers(0, 1 << 32, size=(d_out, words), dtype=np.uint32)
    bits_v = rb.integers(0, 1 << 32, size=(d_in, words), dtype=np.uint32)
    if r % 32:  # bits past r are unused; keep them zero
        keep = np.uint32((1 << (r % 32)) - 1)
        bits_u[:, -1] &= keep
        bits_v[:, -1] &= keep
    rv = np.random.default_rng(3000 + index)
    h = rv.uniform(0.5, 1.5, d_out).astype(np.float32)
    l = rv.uniform(0.5, 1.5, r).astype(np.float32)
    g = rv.uniform(0.5, 1.5, d_in).astype(np.float32)
    x = np.random.default_rng(2000 + index).standard_normal((m, d_in)).astype(np.float32)
    return dict(bits_u=bits_u, bits_v=bits_v, h=h, l=l, g=g, x=x)


# ----------------------------------------------------------------------------- BLR page fixtures

def xorshift_rnd(n: int, seed: int, scale: float) -> np.ndarray:
    """The trainer test's uniform draw in [-scale, scale] (xorshift 13/7/17 on 64 bits)."""
    mask = (1 << 64) - 1
    s = ((seed * 0x9E3779B97F4A7C15) & mask) | 1
    out = np.empty(n, dtype=np.float32)
    for i in range(n):
        s ^= (s << 13) & mask
        s ^= s >> 7
        s ^= (s << 17) & mask
        u = (s >> 11) / float(1 << 53) * 2.0 - 1.0
        out[i] = np.float32(u) * np.float32(scale)
    return out


def pack_sign_bits(signs: np.ndarray) -> np.ndarray:
    """Bitmap [rows][ceil(r/32)] u32 of a sign matrix [rows][r]: bit j of word w <-> index 32w+j, 1 for > 0."""
    signs = np.asarray(signs)
    rows, r = signs.shape
    words = (r + 31) // 32
    pad = np.zeros((rows, words * 32), dtype=np.uint64)
    pad[:, :r] = (signs > 0).astype(np.uint64)
    w = pad.reshape(rows, words, 32) << np.arange(32, dtype=np.uint64)
    return w.sum(axis=2).astype(np.uint32)


def blr_page_inputs(m=256, n=384, r=128, ntok=70, path=0):
    """One path of the trainer's BLR layer test: m = d_out, n = d_in, rank r, ntok tokens."""
    sgn = lambda v: np.where(v >= 0, 1.0, -1.0).astype(np.float32)
    su = sgn(xorshift_rnd(m * r, 10 + path, 1.0)).reshape(m, r)
    sv = sgn(xorshift_rnd(n * r, 20 + path, 1.0)).reshape(n, r)
    h = (np.float32(0.02) + np.abs(xorshift_rnd(m, 30 + path, 0.5)) * np.float32(0.05)).astype(np.float32)
    l = (np.float32(0.5) + np.abs(xorshift_rnd(r, 40 + path, 0.5))).astype(np.float32)
    g = (np.float32(0.1) + np.abs(xorshift_rnd(n, 50 + path, 0.5)) * np.float32(0.2)).astype(np.float32)
    x = xorshift_rnd(ntok * n, 60, 2.0).reshape(ntok, n)
    return dict(bits_u=pack_sign_bits(su), bits_v=pack_sign_bits(sv), h=h, l=l, g=g, x=x)
