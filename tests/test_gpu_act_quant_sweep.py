"""GPU parity over a seeded sweep of Linear shapes for the two paths that
quantize activations: the static-FP8 Linear (act Q + E4M3 x E4M3 GEMM) and
the MXFP4 dynamic-activation Linear (MX act Q + scaled FP4 GEMM).  The
regimes put every launch configuration of their GEMMs under ragged M, N and
K: one/two rows, the 16- and 32-row small-M kernels (with two row blocks),
the split-K path of narrow layers, and the tiled kernels (64 x 64, 128 x 128
and, for the large shapes, 256 x 256 tiles); two more MX regimes with
K % 512 == 0 reach the GEMMs that copy the activations into LDS.  Outputs are compared with the
oracle's fp64 result at the parity bar (relative Frobenius error 1e-2) on
every row up to 512 rows, else on a sample of rows.  WQ_SWEEP_SEED and
WQ_SWEEP_PER_REGIME draw another or a larger sweep."""

import os

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle import gemm as G
from oracle import mx_dynamic as MX
from oracle import quant as Q
from oracle import static_fp8 as S
from weight_only_bit_dequant_amd import synth

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_TOL = 1e-2
REGIMES = [
    ((1, 2), (1024, 4160), (128, 3072)),       # one/two rows
    ((3, 32), (2048, 4160), (128, 3072)),      # 16- and 32-row tiles
    ((33, 64), (1024, 4416), (128, 2048)),     # two row blocks
    ((1, 64), (32, 640), (3200, 8192)),        # narrow layers: split K (K > 3072)
    ((65, 400), (64, 1024), (128, 1536)),      # 64 x 64 tiles
    ((600, 1200), (1024, 2048), (128, 1024)),  # 128 x 128 tiles
    ((3000, 4200), (4000, 4400), (128, 512)),  # 256 x 256 tiles
]
_PER = int(os.environ.get("WQ_SWEEP_PER_REGIME", "2"))
_rng = np.random.RandomState(int(os.environ.get("WQ_SWEEP_SEED", "20261204")))
CASES = []
for _i, (_mr, _nr, _kr) in enumerate(REGIMES):
    for _j in range(_PER):
        for _path in ("static", "mx"):
            CASES.append((_path, int(_rng.randint(_mr[0], _mr[1] + 1)), int(_rng.randint(_nr[0], _nr[1] + 1)),
                          int(_rng.randint(_kr[0], _kr[1] + 1)), 800 + 2 * (_PER * _i + _j) + (_path == "mx")))


# MX regimes with K % 512 == 0, where the MX GEMMs copy the packed activation
# rows and block scales into LDS: the small-M kernel (9 to 64 rows, K up to
# 8192) and the mid-M kernel (65 to 512 rows, N <= 2048: at most 256 tiles of
# 64 x 64, 1024 <= K <= 4096)
MX512_REGIMES = [
    ((9, 64), (512, 4160), (1, 16)),
    ((65, 512), (256, 2048), (2, 8)),
]
MX512_CASES = []
for _i, (_mr, _nr, _kr) in enumerate(MX512_REGIMES):
    for _j in range(_PER):
        MX512_CASES.append((int(_rng.randint(_mr[0], _mr[1] + 1)), int(_rng.randint(_nr[0], _nr[1] + 1)),
                            512 * int(_rng.randint(_kr[0], _kr[1] + 1)), 900 + _PER * _i + _j))


def dev_bf16(bits):
    return synth.as_torch_bf16(bits, DEV)


def host(t):
    return t.detach().cpu().numpy()


def assert_close(Y, ref, what):
    y = C.bf16_to_f32(synth.from_torch_bf16(Y)).astype(np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = G.rel_frobenius(y, ref)
    print(f"[parity] {what}: rel-F {err:.3e}", flush=True)
    assert err <= REL_TOL, f"{what}: rel-F {err}"


@pytest.mark.parametrize("path,M,N,K,cfg", CASES)
def test_act_quant_linear_sweep(path, M, N, K, cfg):
    # shape rules: static K % 16; MXFP4 N, K % 32
    if path == "mx":
        N, K = max(32, N // 32 * 32), max(32, K // 32 * 32)
    else:
        K = max(16, K // 16 * 16)
    W, b, X = synth.linear_case(N, K, M, cfg=cfg, bias=(cfg % 4 < 2))
    print(f"[case] {path} sweep M={M} N={N} K={K} bias={b is not None}", flush=True)
    bd = dev_bf16(b) if b is not None else None
    rows = np.arange(M) if M <= 512 else np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    if path == "static":
        cal = X[: min(M, 32)]
        scale, _ = wq.calibrate_act_scale([dev_bf16(cal)])
        q = wq.quantize("fp8", dev_bf16(W))
        Y = wq.static_fp8_linear(dev_bf16(X), scale, q["codes"], q["scales"], bd)
        torch.cuda.synchronize()
        s_ref = S.scale_from_amax(S.absmax(cal))
        assert host(scale)[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
        wq_ref, ws_ref = Q.quantize_fp8_row(W)
        ref = S.static_linear_fp64(S.quantize_act(X[rows], s_ref), s_ref, wq_ref, ws_ref, b)
    else:
        q = wq.quantize("mxfp4", dev_bf16(W))
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        wq.mxfp4_dynamic_linear(dev_bf16(X), q, bd, out=Y)
        torch.cuda.synchronize()
        wc, ws = Q.quantize_mxfp4(W)
        ref = MX.forward(X[rows], wc, ws, b)
    assert_close(Y[torch.as_tensor(rows, device=DEV)], ref, f"{path} M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K,cfg", MX512_CASES)
def test_mx_lds_kernels_sweep(M, N, K, cfg):
    N = max(32, N // 32 * 32)
    W, b, X = synth.linear_case(N, K, M, cfg=cfg, bias=(cfg % 2 == 0))
    print(f"[case] mx K%512 sweep M={M} N={N} K={K} bias={b is not None}", flush=True)
    bd = dev_bf16(b) if b is not None else None
    q = wq.quantize("mxfp4", dev_bf16(W))
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.mxfp4_dynamic_linear(dev_bf16(X), q, bd, out=Y)
    torch.cuda.synchronize()
    wc, ws = Q.quantize_mxfp4(W)
    assert_close(Y, MX.forward(X, wc, ws, b), f"mx M={M} N={N} K={K}")
