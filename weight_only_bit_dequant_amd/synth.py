"""Seeded synthetic inputs shared by tests, the benchmark and the smoke check.

This module holds no quantization or GEMM arithmetic: it only draws random
tensors with a CPU ``torch.Generator`` and rounds them to bf16 with torch's
own cast, then hands out the bf16 bit patterns (numpy ``uint16``).  Both the
CPU oracle and the HIP path consume exactly these bytes.

Workloads are the pages' toy models: ``nn.Linear(3072, 4096)`` in bf16 with
its default bias and a ``randn(32, 3072)`` bf16 input (every weight-only page,
"Define a linear model ..."), and the two-layer 256 -> 512 -> 128 bias-free
model with ``randn(32, 256)`` inputs ("TorchAO Static FP8 Quantization
(Linear)", "Define a small two-layer Linear model").  ``nn.Linear``'s default
initialisation draws weight and bias from U(-1/sqrt(in), 1/sqrt(in)).
"""

import math

import numpy as np
import torch

# seed bases: weight 1000 + cfg, bias 1001 + cfg, activations 1002 + cfg,
# calibration batch i: 2000 + i
SEED_W, SEED_B, SEED_X, SEED_CAL = 1000, 1001, 1002, 2000

# Linear shape of every weight-only page: in_features K, out_features N
LINEAR_K, LINEAR_N, LINEAR_M = 3072, 4096, 32
MLP_DIMS = (256, 512, 128)
MLP_M = 32
CALIB_STEPS = 10

# The five workloads (C1..C5); M values listed are the ones each one runs at.
WORKLOADS = {
    "int4": dict(fmt="int4", N=LINEAR_N, K=LINEAR_K, M=(32,), bias=True, cfg=1),
    "fp8": dict(fmt="fp8", N=LINEAR_N, K=LINEAR_K, M=(32,), bias=True, cfg=2),
    "nvfp4": dict(fmt="nvfp4", N=LINEAR_N, K=LINEAR_K, M=(32,), bias=True, cfg=3),
    "mxfp4": dict(fmt="mxfp4", N=LINEAR_N, K=LINEAR_K, M=(1, 32, 256, 4096), bias=True, cfg=4),
    "static_fp8": dict(fmt="static_fp8", N=LINEAR_N, K=LINEAR_K, M=(32, 4096), bias=False, cfg=5),
    # the same layer quantized with the asymmetric INT4 scheme (beside the headline configs)
    "int4_asym": dict(fmt="int4_asym", N=LINEAR_N, K=LINEAR_K, M=(32,), bias=True, cfg=7),
}


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _bf16_bits(t):
    return t.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def linear_weight(N, K, seed):
    """bf16 bits [N, K] ~ U(-1/sqrt(K), 1/sqrt(K)) (drawn in fp32, cast to bf16)."""
    b = 1.0 / math.sqrt(K)
    t = torch.empty(N, K, dtype=torch.float32).uniform_(-b, b, generator=_gen(seed))
    return _bf16_bits(t)


def linear_bias(N, K, seed):
    """bf16 bits [N] ~ U(-1/sqrt(K), 1/sqrt(K))."""
    b = 1.0 / math.sqrt(K)
    t = torch.empty(N, dtype=torch.float32).uniform_(-b, b, generator=_gen(seed))
    return _bf16_bits(t)


def activations(M, K, seed):
    """bf16 bits [M, K] ~ N(0, 1)."""
    t = torch.randn(M, K, dtype=torch.float32, generator=_gen(seed))
    return _bf16_bits(t)


def linear_case(N, K, M, cfg, bias=True):
    """(W, b or None, X) for workload number `cfg`."""
    W = linear_weight(N, K, SEED_W + cfg)
    b = linear_bias(N, K, SEED_B + cfg) if bias else None
    X = activations(M, K, SEED_X + cfg)
    return W, b, X


def mlp_weights(dims=MLP_DIMS, cfg=5):
    """Per-layer bf16 weights of the bias-free MLP dims[0] -> dims[1] -> ..."""
    return [linear_weight(dims[i + 1], dims[i], SEED_W + 10 * cfg + i) for i in range(len(dims) - 1)]


def calibration_batches(M, K, steps=CALIB_STEPS):
    return [activations(M, K, SEED_CAL + i) for i in range(steps)]


def special_weight(N, K, seed, kind):
    """Edge-case weights: 'zeros', 'tiny' (values near the bf16 subnormal
    range), 'wide' (per-row magnitudes spread over 2^-20 .. 2^10), 'negzero'
    (all -0.0 except a few entries)."""
    g = _gen(seed)
    if kind == "zeros":
        return np.zeros((N, K), np.uint16)
    if kind == "negzero":
        w = np.full((N, K), 0x8000, np.uint16)
        t = torch.randn(N, K, generator=g)
        mask = torch.rand(N, K, generator=g) < 0.05
        w[mask.numpy()] = _bf16_bits(t)[mask.numpy()]
        return w
    if kind == "tiny":
        t = torch.randn(N, K, generator=g) * 2.0 ** -120
        return _bf16_bits(t)
    if kind == "wide":
        t = torch.randn(N, K, generator=g)
        rows = torch.randint(-20, 11, (N, 1), generator=g).float()
        cols = torch.randint(-6, 7, (1, K), generator=g).float()
        return _bf16_bits(t * torch.exp2(rows) * torch.exp2(cols))
    raise ValueError(kind)


def as_torch_bf16(bits, device=None):
    """uint16 bit array -> torch bfloat16 tensor (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t


def from_torch_bf16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()
