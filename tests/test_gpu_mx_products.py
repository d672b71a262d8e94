"""The scaled E2M1 x E2M1 matrix-core path (MXFP4 page: MX activations x MX
weights) against the closed forms of E2M1 and E8M0, product by product.

Activation row m carries code m % 16 at one K position (7m % K) under block
scale 2^((m / 16) % 16 - 7), zeros elsewhere; weight row n carries code n % 16
at every K position under block scale 2^((n / 16) % 16 - 7).  Without bias,
Y[m][n] is the single product of the two scaled values: at most 4 significant
bits and within bf16's normal range, so the bf16 output must equal it exactly
(a zero product is +0, as the accumulation starts from +0).  The shapes reach
the two small-M kernels (K = 128 and 512), the tiled kernel, the mid-M
kernel (K = 1024) and the 256 x 256 kernel."""

import numpy as np
import pytest
import torch

from oracle import codecs as C

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _pack(codes):
    """Two E2M1 codes per byte along K, the even K in the low nibble."""
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("M,N,K", [(64, 256, 128), (64, 256, 512), (256, 256, 128), (256, 256, 1024), (4096, 3072, 128)])
def test_e2m1_products_exact(M, N, K):
    m, n = np.arange(M), np.arange(N)
    a, b = (m % 16).astype(np.uint8), (n % 16).astype(np.uint8)
    sa, sb = (120 + (m // 16) % 16).astype(np.uint8), (120 + (n // 16) % 16).astype(np.uint8)
    Xc = np.zeros((M, K), dtype=np.uint8)
    Xc[m, (7 * m) % K] = a
    Wc = np.repeat(b[:, None], K, axis=1)
    Xs = np.repeat(sa[:, None], K // 32, axis=1)
    Ws = np.repeat(sb[:, None], K // 32, axis=1)
    va = C.e2m1_decode(a).astype(np.float64) * C.e8m0_decode(sa).astype(np.float64)
    vb = C.e2m1_decode(b).astype(np.float64) * C.e8m0_decode(sb).astype(np.float64)
    ref = np.outer(va, vb) + 0.0
    ref_bits = C.f64_to_bf16(ref)
    assert np.array_equal(C.bf16_to_f32(ref_bits).astype(np.float64), ref), "products are exact in bf16"
    print(f"[case] e2m1 products M={M} N={N} K={K}", flush=True)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    wq.wq_mx_linear(dev(_pack(Xc)), dev(Xs), K, dev(_pack(Wc)), dev(Ws), None, N, Y)
    torch.cuda.synchronize()
    got = Y.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != ref_bits)
    assert bad.size == 0, f"{len(bad)} products differ, first at {bad[:3].tolist()}"
