"""The per-element bound of the GPU output checks (tests/elementwise_bound.py)
is tight enough to catch plausible mistakes: outputs built from the oracle
with a mistake planted in it must fail the check against the correct oracle,
and the correct oracle's own outputs, rounded to bf16, must pass.  Planted:
a dropped bias, one weight's sign flipped (the one with the largest |x w| of
its column), one block scale doubled, and two output columns swapped."""

import numpy as np
import pytest

import elementwise_bound as EB
from oracle import codecs as C
from oracle import gemm as G
from oracle import quant as Q
from weight_only_bit_dequant_amd import synth

F32 = np.float32
FMTS = ["int4", "fp8", "nvfp4", "mxfp4", "int4_asym"]
BLOCK = {"int4": 128, "int4_asym": 128, "nvfp4": 16, "mxfp4": 32}


def _case(fmt):
    M, N, K = 8, 64, 512
    W, b, X = synth.linear_case(N, K, M, cfg=7)
    codes, scales, g = Q.quantize(fmt, W)
    D = Q.dequant(fmt, codes, scales, g)
    return X, b, codes, scales, g, D, G.linear_fp64(X, D, b)


def _as_output(ref):
    return C.f32_to_bf16(np.asarray(ref, np.float64).astype(F32))


def _fails(fmt, y, X, b, codes, scales, g, ref):
    ok, ratio, _ = EB.check(fmt, y, X, codes, scales, g, b, ref)
    return (not ok) and ratio > 1.5


@pytest.mark.parametrize("fmt", FMTS)
def test_correct_outputs_pass(fmt):
    X, b, codes, scales, g, D, ref = _case(fmt)
    ok, ratio, _ = EB.check(fmt, _as_output(ref), X, codes, scales, g, b, ref)
    assert ok and ratio <= 0.55


@pytest.mark.parametrize("fmt", FMTS)
def test_dropped_bias_fails(fmt):
    X, b, codes, scales, g, D, ref = _case(fmt)
    y = _as_output(G.linear_fp64(X, D, None))
    assert _fails(fmt, y, X, b, codes, scales, g, ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_flipped_weight_sign_fails(fmt):
    X, b, codes, scales, g, D, ref = _case(fmt)
    x = np.abs(C.bf16_to_f32(X)).astype(np.float64)
    k = int(np.argmax(x.max(axis=0) * np.abs(D[5])))
    D2 = D.copy()
    D2[5, k] = -D2[5, k]
    assert _fails(fmt, _as_output(G.linear_fp64(X, D2, b)), X, b, codes, scales, g, ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_doubled_block_scale_fails(fmt):
    # the scale that covers K 128 .. of row 9: its 128-K group (INT4), 16- or
    # 32-K block (NVFP4, MXFP4), or the whole row (E4M3 row scale)
    X, b, codes, scales, g, D, ref = _case(fmt)
    D2 = D.copy()
    if fmt == "fp8":
        D2[9, :] *= 2.0
    else:
        D2[9, 128:128 + BLOCK[fmt]] *= 2.0
    assert _fails(fmt, _as_output(G.linear_fp64(X, D2, b)), X, b, codes, scales, g, ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_swapped_columns_fail(fmt):
    X, b, codes, scales, g, D, ref = _case(fmt)
    y = _as_output(ref[:, [1, 0] + list(range(2, ref.shape[1]))])
    assert _fails(fmt, y, X, b, codes, scales, g, ref)


def test_ulp_bf16():
    assert EB.ulp_bf16(1.0) == 2.0 ** -7
    assert EB.ulp_bf16(1.5) == 2.0 ** -7
    assert EB.ulp_bf16(-0.75) == 2.0 ** -8
    assert EB.ulp_bf16(0.0) == 0.0
