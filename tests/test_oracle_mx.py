"""Pins for the MXFP4 dynamic-activation oracle (oracle/mx_dynamic.py).

The activation quantizer reuses the MXFP4 weight rule; these tests pin it on
activations directly (hand-worked blocks whose codes change under the
plausible mistakes: wrong exponent offset, ties away from zero, unsigned zero,
no saturation) and pin the MX GEMM by an exact round trip: operands built on
the MX grid quantize losslessly, so the MX Linear must equal the plain product
to the last bit, which fails for a scale applied to the wrong block, row or
operand.
"""

import numpy as np

from oracle import codecs as C
from oracle import mx_dynamic as MX
from oracle import quant as Q


def bf16(vals):
    return C.f32_to_bf16(np.asarray(vals, np.float32))


def test_quantize_act_hand_blocks():
    row = np.zeros(96, np.float32)
    row[0], row[1] = 0.3, -1.7           # block 0: amax 1.703125 -> e = -2 (scale code 125)
    row[32], row[33], row[34] = 5.0, -0.0, 2.5  # block 1: amax 5 -> e = 0; 5 -> 4 and 2.5 -> 2 (ties to even)
    x = bf16(row)[None, :]
    codes, scales = MX.quantize_act(x)
    assert scales.tolist() == [[125, 127, 0]]  # all-zero block 2 -> e = -127
    # 0.30078125 / 0.25 = 1.203 -> 1.0 (code 2); -1.703 / 0.25 = -6.81 -> saturates to -6 (0xF)
    assert codes[0, 0] == 0x2 and codes[0, 1] == 0xF
    assert codes[0, 32] == 0x6 and codes[0, 33] == 0x8 and codes[0, 34] == 0x4
    assert (codes[0, 2:32] == 0).all() and (codes[0, 64:] == 0).all()


def test_quantize_act_rows_are_independent_and_m_is_free():
    rng = np.random.default_rng(3)
    x = bf16(rng.standard_normal((5, 64)).astype(np.float32))  # M = 5 is not a multiple of 32
    c, s = MX.quantize_act(x)
    c2, s2 = MX.quantize_act(x[::-1].copy())
    assert np.array_equal(c2, c[::-1]) and np.array_equal(s2, s[::-1])


def _mx_grid(rng, rows, k):
    """Values exactly on the MX grid: each 32-block has random E2M1 codes (one
    of them +-6 so the block's exponent is reproduced) times 2^e."""
    codes = rng.integers(0, 16, size=(rows, k)).astype(np.uint8)
    codes[:, ::32] = rng.choice([0x7, 0xF], size=(rows, k // 32))
    e = rng.integers(-6, 4, size=(rows, k // 32))
    vals = C.e2m1_decode(codes) * np.exp2(np.repeat(e, 32, axis=1))
    return bf16(vals), codes, (e + 127).astype(np.uint8)


def test_mx_round_trip_and_exact_linear():
    rng = np.random.default_rng(11)
    X, xcodes, xscales = _mx_grid(rng, 7, 128)
    W, wcodes, wscales = _mx_grid(rng, 32, 128)
    c, s = MX.quantize_act(X)
    assert np.array_equal(s, xscales)
    assert np.array_equal(c, xcodes)  # including negative zeros
    wc, ws = Q.quantize_mxfp4(W)
    assert np.array_equal(wc, wcodes) and np.array_equal(ws, wscales)
    b = bf16(rng.standard_normal(32).astype(np.float32))
    y = MX.forward(X, wc, ws, b)
    exact = C.bf16_to_f32(X).astype(np.float64) @ C.bf16_to_f32(W).astype(np.float64).T
    exact += C.bf16_to_f32(b).astype(np.float64)[None, :]
    assert np.array_equal(y, exact)


def test_mx_linear_brute_force():
    rng = np.random.default_rng(5)
    X = bf16(rng.standard_normal((2, 64)).astype(np.float32))
    W = bf16((rng.standard_normal((32, 64)) * 0.1).astype(np.float32))
    xc, xs = MX.quantize_act(X)
    wc, ws = Q.quantize_mxfp4(W)
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]

    def val(code, scale):
        v = table[int(code) & 7] * 2.0 ** (int(scale) - 127)
        return -v if int(code) & 8 else v

    y = MX.linear_fp64(xc, xs, wc, ws)
    for m in range(2):
        for n in range(32):
            acc = 0.0
            for k in range(64):
                acc += val(xc[m, k], xs[m, k // 32]) * val(wc[n, k], ws[n, k // 32])
            assert acc == y[m, n]
