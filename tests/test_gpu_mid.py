"""GPU parity of the mid-M dequant-GEMM (more than 128 rows, up to 768 tiles of
64 x 64, K % 128 == 0, 1024 <= K <= 16384): 8 waves of a workgroup split K
and meet once in an LDS reduction; activations go straight into LDS, packed
weights straight into registers.

Cases: the edges of the plan (129 rows; 768 tiles), ragged M and N inside the
last tile (N % 64 != 0, and N % 8 != 0 for the element-wise stores), every
unroll depth of the block loop (1, 3, 8 and 16 K blocks per wave, the last a
rolled loop), no bias, both weight layouts, a repeated call (fixed-order
reduction), and the decode pinned element by element with an identity block
as the activations.  Bar: relative Frobenius error 1e-2 against the oracle's
fp64 result on the dequantized weight; the decode bit for bit.
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
REL_TOL = 1e-2
FMTS = ["int4", "fp8", "nvfp4", "mxfp4", "int4_asym"]
# smallest N step each format's scales allow in the rows layout
N_STEP = {"int4": 1, "int4_asym": 1, "fp8": 1, "nvfp4": 16, "mxfp4": 32}


def _run(fmt, M, N, K, cfg, bias=True, layout=wq.LAYOUT_ROWS, rows=None):
    W, b, X = synth.linear_case(N, K, M, cfg=cfg, bias=bias)
    print(f"[case] mid fmt={fmt} M={M} N={N} K={K} bias={bias} layout={layout}", flush=True)
    q = wq.quantize(fmt, synth.as_torch_bf16(W, DEV))
    if layout == wq.LAYOUT_TILES:
        q = wq.repack(q, layout)
    Xd = synth.as_torch_bf16(X, DEV)
    bd = None if b is None else synth.as_torch_bf16(b, DEV)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.linear(Xd, q, bd, out=Y)
    Y2 = wq.linear(Xd, q, bd)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), "repeated call differs"
    codes, scales, g = Q.quantize(fmt, W)
    sel = np.arange(M) if rows is None else rows
    ref = G.linear_fp64(X[sel], Q.dequant(fmt, codes, scales, g), b)
    y = C.bf16_to_f32(synth.from_torch_bf16(Y)).astype(np.float64)[sel]
    assert np.isfinite(y).all(), "non-finite output (unwritten tile?)"
    err = G.rel_frobenius(y, ref)
    print(f"[parity] mid {fmt} M={M} N={N} K={K}: rel-F {err:.3e}", flush=True)
    assert err <= REL_TOL
    return Y


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [
    (129, 4096, 3072),   # first row count of the plan; 3 K blocks per wave, last row tile holds one row
    (200, 1000, 1024),   # ragged M and N (N % 64 = 40); 1 block per wave
    (300, 2048, 8192),   # 8 blocks per wave (the largest unrolled loop)
    (160, 512, 16384),   # 16 blocks per wave (rolled loop)
    (130, 1004, 2048),   # N % 8 = 4: element-wise stores in the last tile
])
def test_mid_parity_rows_layout(fmt, M, N, K):
    step = N_STEP[fmt]
    N = (N + step - 1) // step * step
    _run(fmt, M, N, K, cfg=300 + M % 37)


@pytest.mark.parametrize("fmt", FMTS)
def test_mid_no_bias(fmt):
    _run(fmt, 256, 1024, 2048, cfg=341, bias=False)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(256, 4096, 3072), (200, 1056, 1024)])
def test_mid_tile_layout_same_bits(fmt, M, N, K):
    Yt = _run(fmt, M, N, K, cfg=350, layout=wq.LAYOUT_TILES)
    Yr = _run(fmt, M, N, K, cfg=350, layout=wq.LAYOUT_ROWS)
    assert torch.equal(Yt.view(torch.int16), Yr.view(torch.int16))


@pytest.mark.parametrize("fmt", FMTS)
def test_mid_768_tiles_sampled(fmt):
    # 12 row tiles x 64 column tiles: three workgroups per CU; sampled rows
    M = 768
    _run(fmt, M, 4096, 3072, cfg=360, layout=wq.LAYOUT_TILES, rows=np.arange(0, M, 23))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("layout", [wq.LAYOUT_ROWS, wq.LAYOUT_TILES])
def test_mid_decode_exact(fmt, layout):
    """Identity activations: output row m is dequantized weight column m, bit
    for bit (MXFP4, NVFP4 and E4M3 decode exactly to bf16; INT4 is bf16(code *
    s), the oracle's bf16 dequantized weight)."""
    M, N, K = 256, 2048, 1024
    W = synth.linear_weight(N, K, synth.SEED_W + 370)
    codes, scales, g = Q.quantize(fmt, W)
    want = Q.dequant_bf16(fmt, codes, scales, g)[:, :M].T.copy()
    want[want == 0x8000] = 0  # a -0 weight gives +0: the sum starts from +0
    X = np.zeros((M, K), dtype=np.uint16)
    X[np.arange(M), np.arange(M)] = 0x3F80
    print(f"[case] mid decode {fmt} layout={layout}", flush=True)
    q = wq.quantize(fmt, synth.as_torch_bf16(W, DEV))
    if layout == wq.LAYOUT_TILES:
        q = wq.repack(q, layout)
    Y = wq.linear(synth.as_torch_bf16(X, DEV), q, None)
    torch.cuda.synchronize()
    got = synth.from_torch_bf16(Y)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first at {bad[:3].tolist()}"
