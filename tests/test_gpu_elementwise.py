"""Every output element of the dequant-GEMM against the oracle, within the
per-element bound of tests/elementwise_bound.py (one bf16 ulp of the exact
result plus a first-order fp32 accumulation term, and INT4's bf16 weight
rounding above 128 rows).  The relative Frobenius bar of the parity tests
checks the outputs as a whole; this checks each one, at the benchmark's full
size and in the other launch configurations: one and two rows (operand
loads straight from memory), 32 rows (the benchmark's 16-row blocks, both
layouts), 100 rows on a wide layer (64-column tiles), 256 rows (the mid-M
kernel), 24 rows over a long K (two passes of the waves' K steps), a split-K
narrow layer, and sampled rows at M = 4096 (256 x 256 tiles).  The worst ratio |y - ref| / bound is printed per case."""

import numpy as np
import pytest
import torch

import elementwise_bound as EB
from oracle import gemm as G
from oracle import quant as Q
from weight_only_bit_dequant_amd import synth

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FMTS = ["int4", "fp8", "nvfp4", "mxfp4", "int4_asym"]


def _check(fmt, M, N, K, cfg, layout=wq.LAYOUT_TILES, rows=None, bias=True):
    W, b, X = synth.linear_case(N, K, M, cfg=cfg, bias=bias)
    print(f"[case] elementwise fmt={fmt} M={M} N={N} K={K} layout={layout}", flush=True)
    q = wq.quantize(fmt, synth.as_torch_bf16(W, DEV), layout=layout)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.linear(synth.as_torch_bf16(X, DEV), q, None if b is None else synth.as_torch_bf16(b, DEV), out=Y)
    torch.cuda.synchronize()
    sel = np.arange(M) if rows is None else rows
    codes, scales, g = Q.quantize(fmt, W)
    ref = G.linear_fp64(X[sel], Q.dequant(fmt, codes, scales, g), b)
    y = synth.from_torch_bf16(Y)[sel]
    ok, ratio, worst = EB.check(fmt, y, X[sel], codes, scales, g, b, ref)
    print(f"[elementwise] {fmt} M={M} N={N} K={K}: worst |y-ref|/bound {ratio:.3f} at {worst}", flush=True)
    assert ok, f"{fmt} M={M}: element {worst} exceeds its bound by {ratio:.2f}x"


@pytest.mark.parametrize("fmt", FMTS)
def test_elementwise_full_size_m32(fmt):
    _check(fmt, 32, 4096, 3072, cfg=synth.WORKLOADS[fmt]["cfg"])


@pytest.mark.parametrize("fmt", FMTS)
def test_elementwise_m32_rows_layout(fmt):
    _check(fmt, 32, 4096, 3072, cfg=synth.WORKLOADS[fmt]["cfg"], layout=wq.LAYOUT_ROWS)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 100, 256])
def test_elementwise_other_row_counts(fmt, M):
    _check(fmt, M, 4096, 3072, cfg=400 + M)


@pytest.mark.parametrize("fmt", FMTS)
def test_elementwise_m24_long_k(fmt):
    # 16-row blocks in tile order, the waves' K steps in two passes
    _check(fmt, 24, 4096, 6144, cfg=415)


@pytest.mark.parametrize("fmt", FMTS)
def test_elementwise_split_k_narrow(fmt):
    _check(fmt, 24, 512, 8192, cfg=410, layout=wq.LAYOUT_ROWS, bias=False)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_elementwise_m4096_sampled_rows(fmt):
    M = 4096
    _check(fmt, M, 4096, 3072, cfg=420, rows=np.arange(0, M, 61))
