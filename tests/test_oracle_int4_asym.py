"""Pins for the asymmetric INT4 oracle (oracle.quant.quantize_int4_asym).

Hand-worked groups (codes, scale bits and zero-points written out below were
computed by hand from the stated reading) catch the plausible mistakes: a
divisor of 16, a range that does not include zero, rounding half away from
zero, a zero-point from the unrounded scale.  Brute force checks that every
code is the nearest representable value for the group's (s, z).
"""

import numpy as np

from oracle import codecs as C
from oracle import quant as Q


def bf16(vals):
    return C.f32_to_bf16(np.asarray(vals, np.float32))


def test_hand_worked_groups():
    w = np.zeros((1, 512), np.float32)
    w[0, 0], w[0, 1] = -0.3, 0.5                     # group 0: lo = -0.30078125, hi = 0.5
    w[0, 128:256] = 0.25; w[0, 129] = 0.75           # group 1: all positive -> lo = 0
    w[0, 384:512] = -0.5; w[0, 384] = -1.0           # group 3: all negative -> hi = 0; group 2 all zero
    codes, scales, zeros = Q.quantize_int4_asym(bf16(w))
    # s0 = bf16(0.80078125 / 15) = 219/128 * 2^-5; z0 = rint(0.30078125 / s0 = 5.6256) = 6
    # s1 = bf16(0.75 / 15) = 205/128 * 2^-5;     z1 = 0
    # s3 = bf16(1 / 15) = 137/128 * 2^-4;        z3 = rint(14.949) = 15
    assert scales.tolist() == [[0x3D5B, 0x3D4D, 0x0000, 0x3D89]]
    assert zeros.tolist() == [[6, 0, 0, 15]]
    assert codes[0, 0] == 0 and codes[0, 1] == 15 and (codes[0, 2:128] == 6).all()
    assert codes[0, 128] == 5 and codes[0, 129] == 15 and (codes[0, 130:256] == 5).all()
    assert (codes[0, 256:384] == 0).all()
    assert codes[0, 384] == 0 and (codes[0, 385:512] == 8).all()


def test_codes_are_nearest_and_zero_is_exact():
    rng = np.random.default_rng(17)
    W = bf16(rng.standard_normal((16, 256)).astype(np.float32) * np.float32(0.05) + np.float32(0.01))
    codes, scales, zeros = Q.quantize_int4_asym(W)
    w = C.bf16_to_f32(W).astype(np.float64)
    s = C.bf16_to_f32(scales).astype(np.float64)
    grid = np.arange(16)
    for n in range(16):
        for g in range(2):
            vals = (grid - int(zeros[n, g])) * s[n, g]
            assert 0 <= zeros[n, g] <= 15
            for k in range(g * 128, (g + 1) * 128):
                d = np.abs(vals - w[n, k])
                best = d.min()
                # the chosen code is a nearest value (ties may go either way)
                assert d[codes[n, k]] <= best + 1e-12 * abs(w[n, k]) + 1e-300
    # a zero weight dequantizes to exactly zero
    W0 = W.copy()
    W0[:, 5] = 0
    c0, s0, z0 = Q.quantize_int4_asym(W0)
    assert (Q.dequant_int4_asym(c0, s0, z0)[:, 5] == 0).all()


def test_dequant_and_bf16_form():
    rng = np.random.default_rng(2)
    W = bf16(rng.uniform(-0.02, 0.03, size=(8, 256)).astype(np.float32))
    c, s, z = Q.quantize_int4_asym(W)
    d = Q.dequant_int4_asym(c, s, z)
    err = np.abs(d - C.bf16_to_f32(W).astype(np.float64))
    smax = np.repeat(C.bf16_to_f32(s).astype(np.float64), 128, axis=1)
    assert (err <= smax * 0.5 + 1e-12).all()  # the range [lo, hi] is covered, so no clipping beyond s/2
    b = Q.dequant_bf16("int4_asym", c, (s, z))
    assert np.array_equal(b, C.f32_to_bf16(d.astype(np.float32)))
    assert np.array_equal(Q.int4_asym_scale_words(s, z) & 0xFFFF, s.astype(np.uint32))
