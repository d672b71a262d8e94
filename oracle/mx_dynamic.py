"""MXFP4 dynamic-activation x MXFP4-weight Linear (CPU oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"TorchAO MXFP4 Dynamic Activation + MX Weight (Linear)", intro and title: the
weights are quantized to MXFP4 once; the activations are quantized to MX on
every forward ("dynamic"); on hardware with native MXFP4 matrix units the GEMM
then multiplies the two MX operands directly.

Readings where the page is silent:
  * the activations use the same MXFP4 format and rule as the weights
    (``quant.quantize_mxfp4``): E2M1 codes, one E8M0 scale per 32 consecutive K
    of one row, e = floor(log2 max|x|) - 2 clamped to [-127, 127], codes
    E2M1(clamp(x / 2^e, +-6)) rounded to nearest even with the sign kept;
  * any number of rows M (only K % 32 is needed for the activation blocks);
  * the products of the two dequantized operands are summed exactly (fp64
    here), the bf16 bias is added, and the output is rounded once to bf16.
"""

import numpy as np

from .codecs import bf16_to_f32
from .quant import dequant_mxfp4, mx_blocks


def quantize_act(X_bf16):
    """Dynamic MX quantization of activations X [M, K] (uint16 bf16 bits).
    Returns (codes uint8 [M, K], scales uint8 E8M0 [M, K/32])."""
    return mx_blocks(bf16_to_f32(X_bf16))


def linear_fp64(x_codes, x_scales, w_codes, w_scales, bias_bf16=None):
    """Y = deq(Xq) . deq(Wq)^T (+ b) in fp64 (every dequantized value is exact).
    Returns float64 [M, N]."""
    x = dequant_mxfp4(x_codes, x_scales)
    w = dequant_mxfp4(w_codes, w_scales)
    y = x @ w.T
    if bias_bf16 is not None:
        y = y + bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return y


def forward(X_bf16, w_codes, w_scales, bias_bf16=None):
    """quantize_act then linear_fp64: the page's forward on the quantized model."""
    xc, xs = quantize_act(X_bf16)
    return linear_fp64(xc, xs, w_codes, w_scales, bias_bf16)
