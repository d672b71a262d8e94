"""The fused two-layer static-FP8 MLP (wq_fp8_static_mlp2) against the oracle's
quantized model and against two unfused wq_fp8_static_linear calls."""

import os

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle import gemm as G
from oracle import quant as Q
from oracle import static_fp8 as S
from weight_only_bit_dequant_amd import synth

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev_bf16(bits):
    return synth.as_torch_bf16(bits, DEV)


def rel(Y, ref):
    return G.rel_frobenius(C.bf16_to_f32(synth.from_torch_bf16(Y)).astype(np.float64), ref)


def run_case(M, K1, N1, N2, bias, seed):
    W1 = synth.linear_weight(N1, K1, seed)
    W2 = synth.linear_weight(N2, N1, seed + 1)
    b1 = synth.linear_bias(N1, K1, seed + 2) if bias else None
    b2 = synth.linear_bias(N2, N1, seed + 3) if bias else None
    X = synth.activations(M, K1, seed + 4)
    # scales: layer 1 from X itself; layer 2 from the float model's hidden layer
    s1 = S.scale_from_amax(S.absmax(X))
    h_float = G.to_bf16(G.linear_fp64(X, C.bf16_to_f32(W1).astype(np.float64), b1))
    s2 = S.scale_from_amax(S.absmax(h_float))
    q1, q2 = Q.quantize_fp8_row(W1), Q.quantize_fp8_row(W2)
    print(f"[case] mlp2 M={M} K1={K1} N1={N1} N2={N2} bias={bias}", flush=True)
    t_s1 = torch.tensor([s1], dtype=torch.float32, device=DEV)
    t_s2 = torch.tensor([s2], dtype=torch.float32, device=DEV)
    W1q, w1s = torch.as_tensor(q1[0], device=DEV), torch.as_tensor(q1[1], device=DEV)
    W2q, w2s = torch.as_tensor(q2[0], device=DEV), torch.as_tensor(q2[1], device=DEV)
    tb1 = dev_bf16(b1) if bias else None
    tb2 = dev_bf16(b2) if bias else None
    Xd = dev_bf16(X)
    Y = torch.full((M, N2), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.wq_fp8_static_mlp2(Xd, t_s1, W1q, w1s, tb1, t_s2, W2q, w2s, tb2, Y)
    H = wq.static_fp8_linear(Xd, t_s1, W1q, w1s, tb1)
    Y2 = wq.static_fp8_linear(H, t_s2, W2q, w2s, tb2)
    torch.cuda.synchronize()
    # oracle: the same two static layers with the oracle's own hidden layer
    h_ref = G.to_bf16(S.static_linear_fp64(S.quantize_act(X, s1), s1, q1[0], q1[1], b1))
    y_ref = S.static_linear_fp64(S.quantize_act(h_ref, s2), s2, q2[0], q2[1], b2)
    e_fused, e_unfused = rel(Y, y_ref), rel(Y2, y_ref)
    same = float((Y.view(torch.int16) == Y2.view(torch.int16)).float().mean())
    print(f"[parity] mlp2 fused rel-F {e_fused:.3e}, unfused {e_unfused:.3e}, identical outputs {same:.3f}", flush=True)
    assert e_fused <= 1e-2 and e_unfused <= 1e-2
    assert rel(Y, C.bf16_to_f32(synth.from_torch_bf16(Y2)).astype(np.float64)) <= 1e-2


def test_page_mlp():
    """The page's model at its batch: 32 x 256 -> 512 -> 128, no bias."""
    run_case(32, 256, 512, 128, False, 700)


# single-pass kernel (K1 <= 256, N1 <= 512, N2 <= 128): ragged rows, a ragged
# second K slice of layer 2, the largest shape; looped kernel: everything else
@pytest.mark.parametrize("M,K1,N1,N2,bias", [(20, 96, 80, 40, True), (33, 240, 272, 112, True),
                                              (17, 256, 512, 128, True), (1, 3072, 512, 256, True),
                                              (16, 272, 256, 64, False), (64, 512, 1024, 100, False)])
def test_ragged_and_deep(M, K1, N1, N2, bias):
    run_case(M, K1, N1, N2, bias, 710 + M)


# seeded sweep over both kernel forms: about a third of the shapes fit the
# single-pass kernel (K1 <= 256, N1 <= 512, N2 <= 128), the rest loop; M spans
# one to several row blocks of 16.  WQ_SWEEP_SEED / WQ_SWEEP_PER_REGIME draw
# another or a larger sweep.
_PER = int(os.environ.get("WQ_SWEEP_PER_REGIME", "3"))
_rng = np.random.RandomState(int(os.environ.get("WQ_SWEEP_SEED", "20261205")))
SWEEP = []
for _lim in [(256, 512, 128), (1024, 1024, 384), (2048, 2048, 64)]:
    for _j in range(_PER):
        SWEEP.append((int(_rng.randint(1, 200)), 16 * int(_rng.randint(1, _lim[0] // 16 + 1)),
                      16 * int(_rng.randint(1, _lim[1] // 16 + 1)), int(_rng.randint(1, _lim[2] + 1)),
                      bool(_rng.randint(0, 2))))


@pytest.mark.parametrize("M,K1,N1,N2,bias", SWEEP)
def test_mlp2_sweep(M, K1, N1, N2, bias):
    run_case(M, K1, N1, N2, bias, 900 + M + K1 + N2)
