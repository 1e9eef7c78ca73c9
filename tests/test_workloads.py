"""Checks of the seeded input generators (no arithmetic of the method lives there)."""

import numpy as np

import workloads as wl


def test_lcg_blocked_form_equals_one_step_recurrence():
    for seed in (0x12345678, 0x9E3779B1 ^ (3072 << 8) ^ 3072, 0):
        assert np.array_equal(wl.lcg_codes(seed, 70000), wl.lcg_codes_reference(seed, 70000))


def test_lcg_first_draws_by_hand():
    # state1 = 0x12345678*1664525 + 1013904223 mod 2^32, code = (state >> 16) % 3
    s = 0x12345678
    want = []
    for _ in range(4):
        s = (s * 1664525 + 1013904223) % (1 << 32)
        want.append((s >> 16) % 3)
    assert list(wl.lcg_codes(0x12345678, 4)) == want


def test_pack_puts_first_code_in_low_bits():
    codes = np.ones((1, 128), np.uint8)
    codes[0, 0] = 2
    codes[0, 5] = 0
    codes[0, 127] = 3
    aos = wl.pack_tq2_aos(codes, np.array([[0x3C00]], np.uint16))
    assert aos.size == 34
    assert aos[0] == 0x56          # 01 01 01 10
    assert aos[1] == 0x51          # element 5 (bits 2..3 of byte 1) is 0: 01 01 00 01
    assert aos[31] == 0xD5         # element 127 (bits 6..7 of byte 31) is 3: 11 01 01 01
    assert aos[32] == 0x00 and aos[33] == 0x3C


def test_tiny_workload_shape_and_scales():
    aos, n, k = wl.tiny_weight()
    assert (n, k, aos.size) == (40, 256, 40 * 2 * 34)
    blk = aos.reshape(40, 2, 34)
    d = blk[:, :, 32:34].copy().view("<f2").astype(np.float64)[..., 0]
    assert d[0, 0] == 0.0625 and d[0, 1] == 0.06640625 and d[39, 1] == 0.0625 + 0.0078125 * 39.5
    assert set(np.unique((blk[:, :, :32, None] >> np.array([0, 2, 4, 6], np.uint8)) & 3)) <= {0, 1, 2}


def test_bitmap_packing_order():
    s = -np.ones((1, 64))
    s[0, 0] = 1
    s[0, 33] = 1
    b = wl.pack_sign_bits(s)
    assert b.shape == (1, 2) and b[0, 0] == 1 and b[0, 1] == 2


def test_distribution_workloads_are_deterministic():
    a1, x1 = wl.decode_inputs()
    a2, x2 = wl.decode_inputs()
    assert np.array_equal(a1, a2) and np.array_equal(x1, x2)
    assert a1.size == 4096 * 32 * 34 and x1.shape == (1, 4096)
