"""Static FP8: calibration, activation Q and the FP8 Linear (CPU oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"TorchAO Static FP8 Quantization (Linear)":
  * intro -- observers calibrate the model, then activations and weights are
    quantized to FP8 e4m3; the GEMM can run in FP8 once Q/DQ are fused;
  * "Graph after export (one Linear)" figure -- bf16 activation -> Q -> FP8 ->
    DQ feeds one input of the linear, FP8 weight -> DQ feeds the other;
  * "Calibrate, then insert static FP8 Q/DQ" -- per-tensor activation min/max
    and per-channel weight min/max observed over the calibration forwards,
    baked into the rewritten layer; calibration_steps=10;
  * "Define a small two-layer Linear model" -- Linear(256, 512) then
    Linear(512, 128), both without bias.

Readings where the page is silent: the observers are symmetric (amax =
max(|min|, |max|)); act_scale = fp32(amax / 448); per-channel = per output row
(the FP8-row weight quantizer); the 10 calibration forwards use 10 distinct
batches; layer 2 is calibrated on the float model's bf16 layer-1 output;
activation Q is x / act_scale as an fp32 division, clamped to +-448, rounded
nearest-even to E4M3.
"""

import numpy as np

from .codecs import bf16_to_f32, e4m3_encode, e4m3_decode
from .gemm import linear_fp64, to_bf16
from .quant import quantize_fp8_row

F32 = np.float32


def absmax(X_bf16):
    """max |x| over a bf16 tensor (exact, as fp32)."""
    x = bf16_to_f32(X_bf16)
    return F32(np.abs(x).max()) if x.size else F32(0.0)


def scale_from_amax(amax):
    """act_scale = fp32(amax / 448)."""
    return F32(F32(amax) / F32(448.0))


def quantize_act(X_bf16, act_scale):
    """E4M3(clamp(fp32(x / act_scale), +-448)); act_scale == 0 keeps x (+-0)."""
    x = bf16_to_f32(X_bf16)
    s = F32(act_scale)
    if s > 0:
        q = (x / s).astype(F32)
    else:
        q = x
    return e4m3_encode(np.clip(q, F32(-448.0), F32(448.0)))


def static_linear_fp64(Xq_e4m3, act_scale, Wq_e4m3, w_scale, bias_bf16=None):
    """DQ(x) . DQ(W)^T in fp64: sum_k dec(xq) dec(wq) * act_scale * w_scale[n]
    (+ b).  Returns float64 [M, N]."""
    xd = e4m3_decode(Xq_e4m3) * float(F32(act_scale))
    wd = e4m3_decode(Wq_e4m3) * np.asarray(w_scale, F32).astype(np.float64)[:, None]
    y = xd @ wd.T
    if bias_bf16 is not None:
        y = y + bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return y


def float_forward(X_bf16, weights):
    """The unquantized bf16 model: each layer's output is bf16(fp64 X W^T).
    Returns the list of per-layer inputs and the final bf16 output."""
    inputs = []
    x = X_bf16
    for W in weights:
        inputs.append(x)
        x = to_bf16(linear_fp64(x, bf16_to_f32(W).astype(np.float64)))
    return inputs, x


def calibrate(batches, weights):
    """Per-layer act_scale from absmax observers over the float model's
    forwards on every calibration batch."""
    amax = [F32(0.0)] * len(weights)
    for xb in batches:
        inputs, _ = float_forward(xb, weights)
        for i, xi in enumerate(inputs):
            amax[i] = max(amax[i], absmax(xi))
    return [scale_from_amax(a) for a in amax], amax


def quantize_model(weights):
    """Per-layer (Wq, w_scale) with the FP8-row quantizer."""
    return [quantize_fp8_row(W) for W in weights]


def quant_forward(X_bf16, act_scales, qweights):
    """Quantized model forward: every layer Q(x) -> FP8 linear -> bf16; the
    bf16 output of layer l is the input of layer l + 1.  Returns
    (final fp64 output before its bf16 rounding, list of bf16 layer outputs)."""
    x = X_bf16
    outs = []
    y = None
    for s, (wq, ws) in zip(act_scales, qweights):
        xq = quantize_act(x, s)
        y = static_linear_fp64(xq, s, wq, ws)
        x = to_bf16(y)
        outs.append(x)
    return y, outs
