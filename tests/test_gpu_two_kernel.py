"""The two-kernel DQ -> GEMM form (wq_linear_dq_gemm: "TorchAO FP8 Weight-Only
Quantization (Linear)", intro -- where the DQ is not fused, DQ and GEMM run as
two kernels) against the oracle.

Its weight passes through bf16 (the dequantize-to-bf16 definition, pinned in
the oracle tests) before the product, so two references apply:
  * the oracle's fp64 Linear on the exact dequantized weight, at the common
    bar (relative Frobenius 1e-2);
  * the oracle's fp64 Linear on the oracle's bf16-rounded weight, which the
    GPU result should follow up to its own final bf16 rounding and fp32
    accumulation (relative Frobenius 4e-3, about two bf16 ulps of spread).
The fused kernel's result on the same inputs is also within the common bar.
"""

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle import gemm as G
from oracle import quant as Q
from weight_only_bit_dequant_amd import synth

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FMTS = ["int4", "fp8", "nvfp4", "mxfp4"]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K,layout", [(32, 4096, 3072, 0), (32, 4096, 3072, 1), (256, 1024, 3072, 0),
                                          (16, 256, 4096, 1)])
def test_two_kernel_form_against_the_oracle(fmt, M, N, K, layout):
    print(f"[case] two-kernel fmt={fmt} M={M} N={N} K={K} layout={layout}", flush=True)
    W, b, X = synth.linear_case(N, K, M, cfg=synth.WORKLOADS[fmt]["cfg"] + 40)
    q = wq.quantize(fmt, synth.as_torch_bf16(W, DEV), layout=layout)
    Xd, bd = synth.as_torch_bf16(X, DEV), synth.as_torch_bf16(b, DEV)
    Y2 = wq.linear_two_kernel(Xd, q, bd)
    Y1 = wq.linear(Xd, q, bd)
    torch.cuda.synchronize()
    codes, scales, g = Q.quantize(fmt, W)
    exact = G.linear_fp64(X, Q.dequant(fmt, codes, scales, g), b)
    wbf = C.bf16_to_f32(Q.dequant_bf16(fmt, codes, scales, g)).astype(np.float64)
    via_bf16 = G.linear_fp64(X, wbf, b)
    y2 = C.bf16_to_f32(synth.from_torch_bf16(Y2)).astype(np.float64)
    y1 = C.bf16_to_f32(synth.from_torch_bf16(Y1)).astype(np.float64)
    e_exact, e_bf = G.rel_frobenius(y2, exact), G.rel_frobenius(y2, via_bf16)
    print(f"[parity] two-kernel {fmt}: rel-F {e_exact:.3e} (exact W), {e_bf:.3e} (bf16 W)", flush=True)
    assert np.isfinite(y2).all()
    assert e_exact <= 1e-2 and e_bf <= 4e-3
    assert G.rel_frobenius(y1, exact) <= 1e-2
