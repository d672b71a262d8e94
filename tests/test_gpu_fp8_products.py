"""The E4M3 x E4M3 matrix-core path against the E4M3 closed form, product by
product ("TorchAO Static FP8 Quantization (Linear)": the GEMM runs in FP8).

Activation row m carries code m % 256 at one K position (m % 16) and zeros
elsewhere; weight row n carries code n % 256 at every K position.  With unit
activation and weight scales and no bias, Y[m][n] is then the single product
dec(m % 256) * dec(n % 256), which has at most 8 significant bits and lies
within bf16's normal range, so the bf16 output must equal it exactly.  The two
NaN codes (0x7F, 0xFF) are replaced by zero, and a zero product is +0 (the
accumulation starts from +0).  Three shapes cover the three
kernel families: the small-M kernel (M = 64 row blocks), the tiled kernel
(M = 256) and the 256 x 256 scaled-MFMA kernel (M = 4096, N = 3072)."""

import numpy as np
import pytest
import torch

from oracle import codecs as C

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
K = 16


def _codes(n):
    c = (np.arange(n) % 256).astype(np.uint8)
    c[(c == 0x7F) | (c == 0xFF)] = 0
    return c


@pytest.mark.parametrize("M,N", [(64, 256), (256, 256), (4096, 3072)])
def test_e4m3_products_exact(M, N):
    a, b = _codes(M), _codes(N)
    Xq = np.zeros((M, K), dtype=np.uint8)
    Xq[np.arange(M), np.arange(M) % K] = a
    Wq = np.repeat(b[:, None], K, axis=1)
    # (+ 0.0: a zero product is +0, as the fp32 accumulation from +0 gives it)
    ref = np.outer(C.e4m3_decode(a).astype(np.float64), C.e4m3_decode(b).astype(np.float64)) + 0.0
    ref_bits = C.f64_to_bf16(ref)
    assert np.array_equal(C.bf16_to_f32(ref_bits).astype(np.float64), ref), "products are exact in bf16"
    print(f"[case] e4m3 products M={M} N={N}", flush=True)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    ws_scale = torch.ones(N, dtype=torch.float32, device=DEV)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(1, wq.wq_fp8_linear_workspace(M, N, K)), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_linear(torch.from_numpy(Xq).to(DEV), one, torch.from_numpy(Wq).to(DEV), ws_scale, None, Y, ws)
    torch.cuda.synchronize()
    got = Y.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != ref_bits)
    assert bad.size == 0, f"{len(bad)} products differ, first at {bad[:3].tolist()}"
