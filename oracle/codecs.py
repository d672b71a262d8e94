"""Element codecs: bf16, E4M3 (OCP "fn"), E2M1, E8M0 and 4-bit two's complement.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name the element formats without defining them:
  * "TorchAO NVFP4 Weight-Only Quantization (Linear)", intro: packed FP4 E2M1
    weights, FP8 E4M3 block scales and an FP32 global scale;
  * "TorchAO MXFP4 Dynamic Activation + MX Weight (Linear)", intro: packed
    FP4 E2M1 weights with E8M0 block scales;
  * "TorchAO FP8 Weight-Only Quantization (Linear)" and "TorchAO Static FP8
    Quantization (Linear)", intro: FP8 e4m3;
  * "TorchAO INT4 Weight-Only Quantization (Linear)", intro: 4-bit integer
    codes with zero-point 0.
The value sets below are those formats' published definitions (OCP OFP8 for
E4M3 with no infinities and 0x7F/0xFF as NaN; OCP MX v1.0 for E2M1 and E8M0).

Every encoder takes values that the caller has already clamped to the
format's finite range and rounds to nearest, ties to even, keeping the sign
bit (so -0.0 encodes to the negative-zero code).  Decoders return float64.
"""

import numpy as np

# ---------------------------------------------------------------- bf16 / fp32


def bf16_to_f32(u16):
    """Widen bf16 bit patterns (uint16) exactly to float32: the bf16 bits are
    the top half of the fp32 word."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x):
    """Round float32 values to bf16 (uint16 bit patterns), nearest-even.

    Adding 0x7FFF plus the lowest kept bit to the fp32 word and truncating the
    low 16 bits rounds the (sign-magnitude, monotone) bit pattern to nearest
    with ties going to the even kept pattern; overflow carries into the
    exponent and yields infinity.  NaNs stay quiet NaNs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16), r)
    return r


def f64_to_bf16(x):
    """Round float64 values to bf16 (uint16 bit patterns) in ONE rounding,
    nearest-even: the result is the nearest multiple of the local bf16 spacing
    2^(max(E, -126) - 7) (8 significant bits, fp32's exponent range), ties to
    the even multiple, whose last mantissa bit is 0."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = np.maximum(ex.astype(np.int64) - 1, -126)
    ulp = np.exp2((E - 7).astype(np.float64))
    q = np.rint(a / ulp)
    r = np.copysign(q * ulp, x)
    with np.errstate(over="ignore"):
        r32 = np.where(np.isfinite(x), r, x).astype(np.float32)
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- E4M3 (OCP)

E4M3_MAX = 448.0
E4M3_MIN_SUBNORMAL = 2.0 ** -9
E4M3_MIN_NORMAL = 2.0 ** -6


def e4m3_decode(codes):
    """E4M3 "fn": 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0
    is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN; no infinities."""
    c = np.asarray(codes).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(x):
    """Encode float values with |x| <= 448 to E4M3 codes, nearest-even.

    Subnormal range |x| < 2^-6: the code is round(|x| / 2^-9) (0..8; 8 is the
    smallest normal, whose code is also 8).  Normal range: write
    |x| = 2^E (1 + f), round 8 f to an integer m; m == 8 carries into E.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: input must be clamped to [-448, 448] and not NaN")
    sign = np.signbit(x).astype(np.int64)
    a = np.abs(x)
    sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = ex.astype(np.int64) - 1
    frac = a / np.exp2(E.astype(np.float64)) - 1.0
    m = np.rint(frac * 8.0).astype(np.int64)
    carry = m == 8
    E = np.where(carry, E + 1, E)
    m = np.where(carry, 0, m)
    norm = ((E + 7) << 3) | m
    code = np.where(a < E4M3_MIN_NORMAL, sub, norm)
    return (code | (sign << 7)).astype(np.uint8)


# ---------------------------------------------------------------- E2M1 (MX FP4)

E2M1_MAX = 6.0


def e2m1_decode(codes):
    """E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0 is
    subnormal (0.5 m).  Magnitudes of codes 0..7: 0, .5, 1, 1.5, 2, 3, 4, 6."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = c >> 3
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.exp2((e - 1).astype(np.float64)) * (1.0 + m / 2.0))
    return np.where(s == 1, -mag, mag)


def e2m1_encode(x):
    """Encode float values with |x| <= 6 to 4-bit E2M1 codes (one per uint8),
    nearest-even.  Subnormal range |x| < 1: code round(2|x|) (2 is 1.0, the
    smallest normal).  Normal range: |x| = 2^E (1 + f), m = round(2 f)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)) or np.any(np.abs(x) > E2M1_MAX):
        raise ValueError("e2m1_encode: input must be clamped to [-6, 6] and not NaN")
    sign = np.signbit(x).astype(np.int64)
    a = np.abs(x)
    sub = np.rint(a * 2.0).astype(np.int64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    E = ex.astype(np.int64) - 1
    frac = a / np.exp2(E.astype(np.float64)) - 1.0
    m = np.rint(frac * 2.0).astype(np.int64)
    carry = m == 2
    E = np.where(carry, E + 1, E)
    m = np.where(carry, 0, m)
    norm = ((E + 1) << 1) | m
    code = np.where(a < 1.0, sub, norm)
    return (code | (sign << 3)).astype(np.uint8)


# ---------------------------------------------------------------- E8M0

E8M0_BIAS = 127


def e8m0_decode(codes):
    """E8M0: an unsigned biased exponent; value 2^(c - 127), code 0xFF is NaN."""
    c = np.asarray(codes).astype(np.int64)
    val = np.exp2((c - E8M0_BIAS).astype(np.float64))
    return np.where(c == 0xFF, np.nan, val)


# ---------------------------------------------------------------- INT4


def int4_decode(codes):
    """4-bit two's complement: nibble 0..7 -> 0..7, 8..15 -> -8..-1.
    Accepts nibbles (0..15, uint8) or int8 codes (-8..7)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    return np.where(c >= 8, c - 16, c).astype(np.float64)
