"""Weight quantizers, nibble packing and dequantization (CPU oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Weights follow ``nn.Linear(in_features=K, out_features=N)``: ``W[N, K]`` with
rows contiguous along K.  bf16 tensors are numpy ``uint16`` bit patterns.

Where a page fixes only part of a quantizer, the rest is the plainest reading
that fits it; each such reading is stated in the function's docstring.
"""

import numpy as np

from .codecs import (
    bf16_to_f32,
    f32_to_bf16,
    e4m3_encode,
    e4m3_decode,
    e2m1_encode,
    e2m1_decode,
    e8m0_decode,
    int4_decode,
)

F32 = np.float32

INT4_GROUP = 128
NVFP4_BLOCK = 16
MXFP4_BLOCK = 32


def _div32(a, b):
    """Correctly rounded IEEE fp32 division (numpy float32 arithmetic)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return (np.asarray(a, F32) / np.asarray(b, F32)).astype(F32)


def _mul32(a, b):
    return (np.asarray(a, F32) * np.asarray(b, F32)).astype(F32)


# ------------------------------------------------------------------ INT4


def quantize_int4_sym(W_bf16, group=INT4_GROUP):
    """Symmetric group-wise INT4 ("TorchAO INT4 Weight-Only Quantization
    (Linear)": intro -- symmetric, zero-point 0, because the target's DQ layer
    rejects a nonzero zero-point; "Define a linear model and quantize weights
    to symmetric INT4" -- group_size=128).

    Readings where the page is silent: the group runs over `group` consecutive
    K elements of one output row; scale s = bf16(fp32(max|w| / 7)) (7 is the
    largest positive code, so -8 is never produced); the code divides by the
    bf16-rounded scale so that code * s is exactly the stored dequantized
    value; code = clamp(round_half_even(fp32(w / s)), -8, 7); an all-zero group
    has s = 0 and codes 0.

    Returns (codes int8 [N, K] one code per byte, scales bf16 uint16 [N, K/group]).
    """
    w = bf16_to_f32(W_bf16)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    wg = w.reshape(N, K // group, group)
    amax = np.abs(wg).max(axis=2)
    s_bf16 = f32_to_bf16(_div32(amax, F32(7.0)))
    s = bf16_to_f32(s_bf16)
    q = _div32(wg, s[..., None])
    q = np.where(s[..., None] > 0, q, F32(0.0))
    codes = np.clip(np.rint(q), -8, 7).astype(np.int8).reshape(N, K)
    return codes, s_bf16


def dequant_int4(codes, scales_bf16, group=INT4_GROUP):
    """fp64 dequantized weight: code * s (exact)."""
    c = int4_decode(codes)
    s = bf16_to_f32(scales_bf16).astype(np.float64)
    return c * np.repeat(s, group, axis=1)


def quantize_int4_asym(W_bf16, group=INT4_GROUP):
    """Asymmetric group-wise INT4 with a zero-point ("TorchAO INT4 Weight-Only
    Quantization (Linear)", intro: TorchAO's default int4 weight-only scheme is
    asymmetric, with a nonzero zero-point; the page's own target rejects it and
    uses the symmetric form instead).

    Readings where the page is silent (the usual affine uint4 scheme, groups as
    in the symmetric form): per group of `group` consecutive K of one row,
    lo = min(min w, 0) and hi = max(max w, 0) (the range keeps 0 exactly
    representable); s = bf16(fp32(fp32(hi - lo) / 15)); zero-point
    z = clamp(round_half_even(fp32(-lo / s)), 0, 15); code =
    clamp(round_half_even(fp32(w / s)) + z, 0, 15); dequantized value
    (code - z) * s.  An all-zero group has s = 0, z = 0 and codes 0.

    Returns (codes uint8 [N, K] in 0..15, scales bf16 uint16 [N, K/group],
    zero-points uint8 [N, K/group]).
    """
    w = bf16_to_f32(W_bf16)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    wg = w.reshape(N, K // group, group)
    lo = np.minimum(wg.min(axis=2), F32(0.0))
    hi = np.maximum(wg.max(axis=2), F32(0.0))
    s_bf16 = f32_to_bf16(_div32((hi - lo).astype(F32), F32(15.0)))
    s = bf16_to_f32(s_bf16)
    pos = s > 0
    z = np.where(pos, np.clip(np.rint(_div32(-lo, s)), 0, 15), 0).astype(np.int64)
    q = np.where(pos[..., None], np.rint(_div32(wg, s[..., None])), 0).astype(np.int64)
    codes = np.clip(q + z[..., None], 0, 15).astype(np.uint8).reshape(N, K)
    return codes, s_bf16, z.astype(np.uint8)


def dequant_int4_asym(codes, scales_bf16, zeros, group=INT4_GROUP):
    """fp64 dequantized weight: (code - z) * s (exact)."""
    c = np.asarray(codes, np.int64)
    z = np.repeat(np.asarray(zeros, np.int64), group, axis=1)
    s = np.repeat(bf16_to_f32(scales_bf16).astype(np.float64), group, axis=1)
    return (c - z) * s


def int4_asym_scale_words(scales_bf16, zeros):
    """The library's storage of one group's scale and zero-point: a 32-bit
    word, bf16 scale in bits 0-15 and the zero-point in bits 16-19."""
    return np.asarray(scales_bf16, np.uint32) | (np.asarray(zeros, np.uint32) << 16)


# ------------------------------------------------------------------ FP8 row


def quantize_fp8_row(W_bf16):
    """FP8 E4M3 weight-only ("TorchAO FP8 Weight-Only Quantization (Linear)":
    intro and "Define a linear model and quantize weights to FP8" --
    Float8WeightOnlyConfig with its defaults).

    Reading: one fp32 scale per output row, s = fp32(max|w_row| / 448) (448 is
    the largest finite E4M3 magnitude); code = E4M3(clamp(fp32(w / s), +-448))
    rounded nearest-even; an all-zero row has s = 0 and codes +-0.

    The same rule gives the per-channel weight scales of the static-FP8 path
    ("TorchAO Static FP8 Quantization (Linear)", "Calibrate, then insert static
    FP8 Q/DQ": per-channel weight min/max).

    Returns (codes uint8 [N, K], scales float32 [N]).
    """
    w = bf16_to_f32(W_bf16)
    amax = np.abs(w).max(axis=1)
    s = _div32(amax, F32(448.0))
    q = _div32(w, s[:, None])
    q = np.where(s[:, None] > 0, q, w)
    q = np.clip(q, F32(-448.0), F32(448.0))
    return e4m3_encode(q), s


def dequant_fp8_row(codes, scales):
    return e4m3_decode(codes) * np.asarray(scales, F32).astype(np.float64)[:, None]


# ------------------------------------------------------------------ NVFP4


def quantize_nvfp4(W_bf16, block=NVFP4_BLOCK):
    """NVFP4 ("TorchAO NVFP4 Weight-Only Quantization (Linear)": intro -- packed
    E2M1 weights, E4M3 block scales, an FP32 global scale, two-level
    dequantization; last two weight dims divisible by 16).

    Readings where the page is silent: blocks are 16 consecutive K elements of
    one row; with A = max|W| over the tensor,
      g  = fp32(A / 2688)                      (2688 = 448 * 6)
      t  = fp32(fp32(max|w_block| / 6) / g)
      sc = E4M3(clamp(t, 2^-9, 448))           (the clamp keeps every scale > 0)
      S  = fp32(dec(sc) * g)
      code = E2M1(clamp(fp32(w / S), +-6))
    An all-zero tensor has g = 0: scales clamp to 2^-9 and codes are +-0.

    Returns (codes uint8 [N, K] one 4-bit code per byte, block scales uint8
    E4M3 [N, K/16], global scale float32).
    """
    w = bf16_to_f32(W_bf16)
    N, K = w.shape
    if N % block or K % block:
        raise ValueError("NVFP4 needs N and K divisible by 16")
    A = np.abs(w).max() if w.size else F32(0.0)
    g = _div32(A, F32(2688.0))
    wb = w.reshape(N, K // block, block)
    ab = np.abs(wb).max(axis=2)
    if g > 0:
        t = _div32(_div32(ab, F32(6.0)), g)
    else:
        t = np.zeros_like(ab)
    t = np.clip(t, F32(2.0 ** -9), F32(448.0))
    sc = e4m3_encode(t)
    d = e4m3_decode(sc).astype(F32)
    S = _mul32(d, g)
    q = _div32(wb, S[..., None])
    q = np.where(S[..., None] > 0, q, wb)
    q = np.clip(q, F32(-6.0), F32(6.0))
    codes = e2m1_encode(q).reshape(N, K)
    return codes, sc, F32(g)


def dequant_nvfp4(codes, scales_e4m3, g, block=NVFP4_BLOCK):
    d = np.repeat(e4m3_decode(scales_e4m3), block, axis=1)
    return e2m1_decode(codes) * d * float(F32(g))


# ------------------------------------------------------------------ MXFP4


def quantize_mxfp4(W_bf16, block=MXFP4_BLOCK):
    """MXFP4 ("TorchAO MXFP4 Dynamic Activation + MX Weight (Linear)": intro --
    packed E2M1 weights, E8M0 block scales, block size 32; K and N divisible
    by 32).

    Readings where the page is silent: blocks are 32 consecutive K elements of
    one row; the shared exponent is e = floor(log2(max|w_block|)) - 2 (2 is the
    exponent of E2M1's largest value 6), taken from the binary exponent of the
    fp32 value (not a log2 call) and clamped to [-127, 127]; the scale code is
    e + 127; code = E2M1(clamp(fp32(w / 2^e), +-6)) -- the division is exact,
    and magnitudes in [6, 8) saturate to 6.  An all-zero block gets e = -127
    (code 0) and codes +-0.

    Returns (codes uint8 [N, K], scales uint8 E8M0 [N, K/32]).
    """
    w = bf16_to_f32(W_bf16)
    N, K = w.shape
    if N % block or K % block:
        raise ValueError("MXFP4 needs N and K divisible by 32")
    return mx_blocks(w, block)


def mx_blocks(w, block=MXFP4_BLOCK):
    """The MX quantization steps of ``quantize_mxfp4`` on an fp32 matrix whose
    rows are split into blocks of 32 consecutive elements (K % 32 == 0).
    Returns (codes uint8 [R, K], scales uint8 E8M0 [R, K/32])."""
    N, K = w.shape
    if K % block:
        raise ValueError("MX blocks need K divisible by 32")
    wb = w.reshape(N, K // block, block)
    ab = np.abs(wb).max(axis=2)
    _, ex = np.frexp(np.where(ab > 0, ab, F32(1.0)))
    e = ex.astype(np.int64) - 1 - 2
    e = np.where(ab > 0, e, -127)
    e = np.clip(e, -127, 127)
    scale_code = (e + 127).astype(np.uint8)
    p = np.exp2(e.astype(np.float64)).astype(F32)
    q = _div32(wb, p[..., None])
    q = np.clip(q, F32(-6.0), F32(6.0))
    codes = e2m1_encode(q).reshape(N, K)
    return codes, scale_code


def dequant_mxfp4(codes, scales_e8m0, block=MXFP4_BLOCK):
    return e2m1_decode(codes) * np.repeat(e8m0_decode(scales_e8m0), block, axis=1)


# ------------------------------------------------------------------ packing


def pack_nibbles(codes):
    """Two 4-bit codes per byte along K: byte j of a row holds element 2j in
    its low nibble and element 2j+1 in its high nibble ("TorchAO INT4
    Weight-Only Quantization (Linear)", "Export and compile": one-code-per-byte
    int8 data re-packed into a 4-bit constant; nibble order is this reading)."""
    c = np.asarray(codes).astype(np.uint8) & np.uint8(0xF)
    if c.shape[-1] % 2:
        raise ValueError("the packed axis needs an even length")
    return (c[..., 0::2] | (c[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0xF)
    out[..., 1::2] = p >> np.uint8(4)
    return out


# ------------------------------------------------------------------ dequantize to bf16


def dequant_bf16(fmt, codes, scales, g=None):
    """Dequantize to bf16 (uint16), the two-kernel form's DQ output ("TorchAO
    FP8 Weight-Only Quantization (Linear)", intro: DQ and GEMM may run as two
    kernels).  Definition: evaluate the scale product in fp32 in the order
    code * block-scale (* global), then round once more to bf16:
      int4  : bf16(code * s)                    (exact in fp32)
      int4_asym : bf16((code - z) * s)          (exact in fp32)
      fp8   : bf16(fp32(dec(code) * s))
      nvfp4 : bf16(fp32(fp32(dec(code) * dec(sc)) * g))
      mxfp4 : bf16(fp32(dec(code) * 2^e))
    """
    if fmt == "int4":
        c = int4_decode(codes).astype(F32)
        s = np.repeat(bf16_to_f32(scales), codes.shape[1] // scales.shape[1], axis=1)
        return f32_to_bf16(_mul32(c, s))
    if fmt == "int4_asym":
        sc, z = scales
        c = (np.asarray(codes, np.int64) - np.repeat(np.asarray(z, np.int64), INT4_GROUP, axis=1)).astype(F32)
        s = np.repeat(bf16_to_f32(sc), INT4_GROUP, axis=1)
        return f32_to_bf16(_mul32(c, s))
    if fmt == "fp8":
        c = e4m3_decode(codes).astype(F32)
        return f32_to_bf16(_mul32(c, np.asarray(scales, F32)[:, None]))
    if fmt == "nvfp4":
        c = e2m1_decode(codes).astype(F32)
        d = np.repeat(e4m3_decode(scales).astype(F32), NVFP4_BLOCK, axis=1)
        return f32_to_bf16(_mul32(_mul32(c, d), F32(g)))
    if fmt == "mxfp4":
        c = e2m1_decode(codes).astype(F32)
        p = np.repeat(e8m0_decode(scales).astype(F32), MXFP4_BLOCK, axis=1)
        return f32_to_bf16(_mul32(c, p))
    raise ValueError(fmt)


def quantize(fmt, W_bf16):
    """Dispatch: returns (codes, scales, global_or_None)."""
    if fmt == "int4":
        c, s = quantize_int4_sym(W_bf16)
        return c, s, None
    if fmt == "int4_asym":
        c, s, z = quantize_int4_asym(W_bf16)
        return c, (s, z), None
    if fmt == "fp8":
        c, s = quantize_fp8_row(W_bf16)
        return c, s, None
    if fmt == "nvfp4":
        return quantize_nvfp4(W_bf16)
    if fmt == "mxfp4":
        c, s = quantize_mxfp4(W_bf16)
        return c, s, None
    raise ValueError(fmt)


def dequant(fmt, codes, scales, g=None):
    """Exact fp64 dequantized weight [N, K]."""
    if fmt == "int4":
        return dequant_int4(codes, scales)
    if fmt == "int4_asym":
        return dequant_int4_asym(codes, scales[0], scales[1])
    if fmt == "fp8":
        return dequant_fp8_row(codes, scales)
    if fmt == "nvfp4":
        return dequant_nvfp4(codes, scales, g)
    if fmt == "mxfp4":
        return dequant_mxfp4(codes, scales)
    raise ValueError(fmt)


# ------------------------------------------------------------------ kernel tile order


TILE_ROWS, TILE_BYTES, TILE_K = 16, 64, 128
SCALE_TILE_BYTES = {"int4": 2, "int4_asym": 4, "nvfp4": 8, "mxfp4": 4}


def tile_order(fmt, packed, scales):
    """The kernel tile order of a packed weight and its block scales (the
    one-time re-layout of the packed constant, "TorchAO INT4 Weight-Only
    Quantization (Linear)", "Export and compile").  Layout definition: the
    packed rows are cut into tiles of 16 rows x 64 bytes; tiles are taken
    row group by row group, and within a row group column block by column
    block; a tile stores its 16 rows' 64 bytes one after the other.  The block
    scales of 128 K per row (2, 4, 8 or 4 bytes for INT4, INT4_ASYM, NVFP4,
    MXFP4) follow the same tiles.  FP8 row scales are returned unchanged.

    packed: uint8 [N, row_bytes]; scales: the format's scale array (row-major,
    any dtype).  Returns (packed_t uint8 [N * row_bytes], scales_t uint8 bytes
    or the FP8 float array)."""
    p = np.asarray(packed, np.uint8)
    N, rb = p.shape
    if N % TILE_ROWS or rb % TILE_BYTES:
        raise ValueError("tile order needs N % 16 == 0 and row bytes % 64 == 0")
    out = np.empty(N * rb, np.uint8)
    pos = 0
    for g in range(N // TILE_ROWS):
        for j in range(rb // TILE_BYTES):
            for r in range(TILE_ROWS):
                out[pos:pos + TILE_BYTES] = p[g * TILE_ROWS + r, j * TILE_BYTES:(j + 1) * TILE_BYTES]
                pos += TILE_BYTES
    if fmt == "fp8":
        return out, np.asarray(scales, np.float32)
    sb = SCALE_TILE_BYTES[fmt]
    sbytes = np.ascontiguousarray(scales).view(np.uint8).reshape(N, -1)
    tiles = sbytes.shape[1] // sb
    st = np.empty(sbytes.size, np.uint8)
    pos = 0
    for g in range(N // TILE_ROWS):
        for j in range(tiles):
            for r in range(TILE_ROWS):
                st[pos:pos + sb] = sbytes[g * TILE_ROWS + r, j * sb:(j + 1) * sb]
                pos += sb
    return out, st


def packed_weight(fmt, codes):
    """The byte stream the GEMM reads: nibble-packed for the 4-bit formats,
    the E4M3 code bytes themselves for FP8."""
    if fmt == "fp8":
        return np.asarray(codes, np.uint8)
    return pack_nibbles(codes)
