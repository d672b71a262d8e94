"""Pins for oracle/codecs.py: library casts, format-spec golden values, brute
force and exhaustive tables (no GPU)."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs as C

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), float(val)))
    return rows


def _same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


# ------------------------------------------------------------------ bf16


def test_bf16_widen_matches_torch_view():
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = C.bf16_to_f32(u)
    ref = torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert _same(ours, ref)


def test_f32_to_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 128, 200000))).astype(np.float32)
    # exact ties between adjacent bf16 values, both parities, and specials
    hi = rng.integers(0, 0x7F80, 20000).astype(np.uint32) << 16
    ties = (hi | 0x8000).view(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45, -1e-45], np.float32)
    x = np.concatenate([x, ties, -ties, specials])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C.f32_to_bf16(x), ref)
    assert np.isnan(C.bf16_to_f32(C.f32_to_bf16(np.array([np.nan], np.float32))))[0]


def _bf16_nearest_bruteforce(x):
    """Nearest bf16 by exact rational distance to the two bracketing bf16
    values, ties to the even bit pattern."""
    f = np.float32(x)
    u = int(C.f32_to_bf16(np.array([f]))[0])
    cands = {(u - 1) & 0xFFFF, u, (u + 1) & 0xFFFF}
    best = None
    for c in cands:
        v = float(C.bf16_to_f32(np.array([c], np.uint16))[0])
        if not np.isfinite(v):
            continue
        d = abs(Fraction(v) - Fraction(float(x)))
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_f64_to_bf16_single_rounding():
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(300) * np.exp2(rng.integers(-60, 60, 300)))
    # values that a fp64 -> fp32 -> bf16 double rounding gets wrong: just
    # above a bf16 midpoint by less than half an fp32 ulp
    for _ in range(200):
        a = int(rng.integers(0x3000, 0x4F00))
        lo = float(C.bf16_to_f32(np.array([a], np.uint16))[0])
        hi = float(C.bf16_to_f32(np.array([a + 1], np.uint16))[0])
        mid = (lo + hi) / 2
        xs += [mid, mid * (1 + 2.0 ** -40), mid * (1 - 2.0 ** -40), -mid * (1 + 2.0 ** -40)]
    xs = np.array(xs, np.float64)
    got = C.f64_to_bf16(xs)
    want = np.array([_bf16_nearest_bruteforce(x) if x >= 0 else _bf16_nearest_bruteforce(-x) | 0x8000
                     for x in xs], np.uint16)
    assert np.array_equal(got, want)
    # a near-tie that double rounding would send to the even neighbour below
    lo = float(C.bf16_to_f32(np.array([0x3F80], np.uint16))[0])
    hi = float(C.bf16_to_f32(np.array([0x3F81], np.uint16))[0])
    x = (lo + hi) / 2 * (1 + 2.0 ** -40)
    assert C.f64_to_bf16(np.array([x]))[0] == 0x3F81
    assert C.f32_to_bf16(np.array([x], np.float32))[0] == 0x3F80  # the double-rounding trap


# ------------------------------------------------------------------ E4M3


def test_e4m3_decode_all_codes_vs_torch():
    u = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(u).view(torch.float8_e4m3fn).float().numpy()
    assert _same(C.e4m3_decode(u), ref)


def test_e4m3_decode_spec_values():
    for code, val in _golden("e4m3_specials.txt"):
        assert _same(C.e4m3_decode(np.array([code]))[0], val), hex(code)
    vals = C.e4m3_decode(np.arange(256))
    assert np.isnan(vals).sum() == 2
    assert np.nanmax(vals) == 448.0


def test_e4m3_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = C.e4m3_decode(codes)
    assert np.array_equal(C.e4m3_encode(vals), codes)


def test_e4m3_encode_ties_to_even_and_neighbours():
    pos = np.array([c for c in range(0x7F)], np.int64)
    v = C.e4m3_decode(pos)
    for i in range(len(v) - 1):
        mid = (v[i] + v[i + 1]) / 2
        even = pos[i] if pos[i] % 2 == 0 else pos[i + 1]
        assert C.e4m3_encode(np.array([mid]))[0] == even
        assert C.e4m3_encode(np.array([-mid]))[0] == even | 0x80
        eps = (v[i + 1] - v[i]) * 1e-3
        assert C.e4m3_encode(np.array([mid - eps]))[0] == pos[i]
        assert C.e4m3_encode(np.array([mid + eps]))[0] == pos[i + 1]


def test_e4m3_encode_matches_torch_cast_random():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-12, 9, 200000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(C.e4m3_encode(x), ref)


def test_e4m3_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        C.e4m3_encode(np.array([449.0]))


def test_e4m3_negative_zero_and_tiny():
    assert C.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert C.e4m3_encode(np.array([-(2.0 ** -12)]))[0] == 0x80
    assert C.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00  # tie between 0 and 2^-9 -> even (0)
    assert C.e4m3_encode(np.array([3 * 2.0 ** -10]))[0] == 0x02  # tie 1 vs 2 -> even (2)


# ------------------------------------------------------------------ E2M1


def test_e2m1_decode_vs_spec_table():
    g = _golden("e2m1_values.txt")
    assert len(g) == 16
    for code, val in g:
        assert _same(C.e2m1_decode(np.array([code]))[0], val), hex(code)


def _e2m1_bruteforce(x):
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = abs(x)
    best = min(range(8), key=lambda c: (abs(mags[c] - a), c % 2))
    return best | (8 if np.signbit(x) else 0)


def test_e2m1_encode_ties_from_spec():
    # midpoints between consecutive magnitudes go to the even code
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, code in ties.items():
        assert C.e2m1_encode(np.array([x]))[0] == code, x
        assert C.e2m1_encode(np.array([-x]))[0] == code | 8, x


def test_e2m1_encode_dense_grid_bruteforce():
    grid = np.linspace(-6, 6, 24001)
    # fp32 neighbours of every tie point
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    near = []
    for t in ties:
        for k in range(-4, 5):
            near.append(np.float32(t) + np.float32(k) * np.spacing(np.float32(t)))
    x = np.concatenate([grid, np.array(near, np.float64), -np.array(near, np.float64), [0.0, -0.0, 6.0, -6.0]])
    got = C.e2m1_encode(x)
    want = np.array([_e2m1_bruteforce(v) for v in x], np.uint8)
    assert np.array_equal(got, want)


def test_e2m1_roundtrip():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(C.e2m1_encode(C.e2m1_decode(codes)), codes)


# ------------------------------------------------------------------ E8M0 and INT4


def test_e8m0_decode_vs_torch_and_spec():
    u = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(u).view(torch.float8_e8m0fnu).float().numpy()
    ours = C.e8m0_decode(u)
    assert _same(ours[1:], ref[1:])
    # code 0 is 2^-127, an fp32 subnormal; check it in fp64 against the spec value
    for code, val in _golden("e8m0_specials.txt"):
        assert _same(ours[code], val), hex(code)


def test_int4_twos_complement():
    nib = np.arange(16)
    want = np.array([0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1], np.float64)
    assert np.array_equal(C.int4_decode(nib), want)
    assert np.array_equal(C.int4_decode(np.arange(-8, 8).astype(np.int8)), np.arange(-8, 8))
