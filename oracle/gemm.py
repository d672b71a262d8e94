"""fp64 Linear, error measures and the page's ``sqnr`` helper (CPU oracle).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""

import numpy as np

from .codecs import bf16_to_f32, f64_to_bf16


def linear_fp64(X_bf16, Wdeq, bias_bf16=None):
    """Y = X . Wdeq^T (+ b) in fp64, the ``nn.Linear`` forward of every page's
    toy model ("Define a linear model ..." sections) with the weight replaced
    by its dequantized value (the DQ-prologue-into-GEMM of each intro).

    X_bf16: uint16 [M, K]; Wdeq: float64 [N, K]; bias_bf16: uint16 [N] or None.
    Returns float64 [M, N].  The library matmul is the only step; every input
    is exact in fp64, so the only rounding is fp64 accumulation.
    """
    x = bf16_to_f32(X_bf16).astype(np.float64)
    w = np.asarray(Wdeq, dtype=np.float64)
    if x.shape[1] != w.shape[1]:
        raise ValueError("X and W disagree on K")
    y = x @ w.T
    if bias_bf16 is not None:
        y = y + bf16_to_f32(bias_bf16).astype(np.float64)[None, :]
    return y


def to_bf16(y):
    """Round an fp64 result once to bf16 (uint16), nearest-even."""
    return f64_to_bf16(y)


def rel_frobenius(y, ref):
    """||y - ref||_F / ||ref||_F, evaluated in fp64."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm((y - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return num / den if den > 0 else (0.0 if num == 0 else np.inf)


def sqnr(a, b):
    """Signal-to-quantization-noise ratio in dB as the helper in "TorchAO Static
    FP8 Quantization (Linear)", "Imports" defines it: flatten both, cast to
    fp32, 20 log10(||a|| / max(||a - b||, 1e-12)), evaluated in fp32."""
    a = np.asarray(a, dtype=np.float32).ravel()
    b = np.asarray(b, dtype=np.float32).ravel()
    signal = np.float32(np.sqrt(np.sum(a * a, dtype=np.float32)))
    d = (a - b).astype(np.float32)
    noise = np.float32(np.sqrt(np.sum(d * d, dtype=np.float32)))
    return float(np.float32(20.0) * np.log10(np.float32(signal / max(noise, np.float32(1e-12)))))


def sqnr_fp64(a, b):
    """The same ratio evaluated in fp64 (for error bounds that need it)."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    noise = max(np.linalg.norm(a - b), 1e-12)
    return float(20.0 * np.log10(np.linalg.norm(a) / noise))
