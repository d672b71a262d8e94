"""Per-element error bound for a dequant-GEMM output against the oracle.

The kernels compute Y = bf16(fl32(sum_k x_k * w'_k) * cs + b): bf16 x bf16
products are exact in fp32, the sums run in fp32 in some order, the column
scale (FP8 row scale, NVFP4 global scale) and the bias are applied once, and
the result is rounded to bf16 once.  w' is the decoded weight; for E4M3,
NVFP4 and MXFP4 it is the oracle's dequantized weight divided by the column
scale, exactly.  INT4 has two forms: up to 128 rows the kernels sum each
128-K group as s * (sum x (code + 136) - 136 sum x) (INT4_ASYM: codes offset
by 128 and 128 + z), whose fp32 partial sums grow with the offset; above
that each weight is first rounded to bf16(code * s), an extra relative error
of at most 2^-9 per weight.

Bound per element (first order in the unit roundoff u = 2^-24):
  |y - ref| <= ulp_bf16(ref) + (n + 4) u S_eff + 2^-9 S_int4 + tiny
where ref is the oracle's exact fp64 result, ulp_bf16(ref) one bf16 unit in
the last place of ref (the final rounding takes at most half of it), n the
length of the longest fp32 summation chain (at most K / 8 + 16: the kernels
add 8-element MFMA groups, K steps and at most 16 wave or split partials),
S_eff = |X| . |W_eff|^T + |b| with |W_eff| the magnitudes the fp32 sums
actually see (|w'| * cs, or s * (code + offsets) for INT4), and S_int4 =
|X| . |W|^T for INT4 only (its bf16(code * s) form).  Every term is an upper
bound, so a correct kernel never exceeds it; a wrong block scale, a flipped
code or a dropped bias moves an output by far more than the accumulation
term (the CPU test of this module plants such mistakes in the oracle).
"""

import numpy as np

from oracle import codecs as C
from oracle import quant as Q

U = 2.0 ** -24


def ulp_bf16(x):
    """One bf16 ulp of |x| (0 for 0): 2^(floor(log2|x|) - 7)."""
    a = np.abs(np.asarray(x, np.float64))
    m, e = np.frexp(a)  # a = m 2^e, m in [0.5, 1)
    return np.where(a > 0, np.ldexp(1.0, e - 8), 0.0)


def effective_magnitudes(fmt, codes, scales, g):
    """|W_eff| [N, K] (fp64): what the kernels' fp32 sums accumulate, per
    weight, and the plain |W| (for INT4's bf16 form)."""
    W = np.abs(Q.dequant(fmt, codes, scales, g))
    if fmt == "int4":
        s = np.repeat(C.bf16_to_f32(scales).astype(np.float64), Q.INT4_GROUP, axis=1)
        c = np.asarray(codes, np.float64)
        trick = s * (c + 136.0 + 136.0)
        return np.maximum(trick, W), W
    if fmt == "int4_asym":
        sc, z = scales
        s = np.repeat(C.bf16_to_f32(sc).astype(np.float64), Q.INT4_GROUP, axis=1)
        zz = np.repeat(np.asarray(z, np.float64), Q.INT4_GROUP, axis=1)
        u = np.asarray(codes, np.float64)
        trick = s * ((128.0 + u) + (128.0 + zz))
        return np.maximum(trick, W), W
    return W, None


def bound(fmt, X_bits, codes, scales, g, b_bits, ref):
    """Per-element bound for outputs `ref` (fp64 [rows, N]) of activations
    X_bits (bf16 [rows, K])."""
    x = np.abs(C.bf16_to_f32(X_bits).astype(np.float64))
    K = x.shape[1]
    Weff, Wplain = effective_magnitudes(fmt, codes, scales, g)
    S = x @ Weff.T
    if b_bits is not None:
        S = S + np.abs(C.bf16_to_f32(b_bits).astype(np.float64))[None, :]
    n = K / 8.0 + 16.0
    # (1 + 2^-7): the final rounding also acts on the accumulated error
    bnd = ulp_bf16(ref) + (1.0 + 2.0 ** -7) * (n + 4.0) * U * S + 2.0 ** -126
    if Wplain is not None:
        bnd = bnd + 2.0 ** -9 * (x @ Wplain.T)
    return bnd


def check(fmt, Y_bits, X_bits, codes, scales, g, b_bits, ref):
    """Returns (ok, worst ratio |y - ref| / bound, index of the worst element)."""
    y = C.bf16_to_f32(np.asarray(Y_bits, np.uint16)).astype(np.float64)
    bnd = bound(fmt, X_bits, codes, scales, g, b_bits, ref)
    ratio = np.abs(y - ref) / bnd
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return bool(np.isfinite(y).all() and (ratio <= 1.0).all()), float(ratio[worst]), worst
