"""GPU checks of the kernel tile order (layout 1, include/wq.h "Weight layouts").

* wq_repack: rows -> tiles equals the oracle's tile order of the oracle's
  packed weight and scales, byte for byte, and tiles -> rows gives back the
  canonical bytes (the round trip the layout must satisfy).
* Every kernel that reads a packed weight gives the same bits from either
  layout: the tile order changes only where bytes are fetched, not the
  arithmetic or its order, so Y (and the dequantized weight) must be
  identical.  The launch configurations covered: one/two rows, 16- and 32-row
  no-split tiles, two row blocks, 64-column tiles of 65-128 rows, split K
  with its reduction, the LDS-tiled kernels (64x64 with K groups, 128x128) and
  the 256x256 kernels; the static-FP8 GEMMs; the MX dynamic GEMMs.
* One case per format also meets the oracle bar directly.
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
FMTS = ["int4", "fp8", "nvfp4", "mxfp4", "int4_asym"]
ROWS, TILES = wq.LAYOUT_ROWS, wq.LAYOUT_TILES


def _scale_bytes(q):
    return q["scales"].contiguous().view(torch.uint8).cpu().numpy().ravel()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(64, 256), (96, 640), (4096, 3072)])
def test_repack_matches_oracle_and_round_trips(fmt, N, K):
    if fmt == "mxfp4" and N % 32:
        N += 16
    print(f"[case] repack fmt={fmt} N={N} K={K}", flush=True)
    W = synth.linear_weight(N, K, 700 + N % 97)
    q = wq.quantize(fmt, synth.as_torch_bf16(W, DEV))
    t = wq.repack(q, TILES)
    back = wq.repack(dict(t), ROWS)
    torch.cuda.synchronize()
    codes, scales, _ = Q.quantize(fmt, W)
    if fmt == "int4_asym":
        scales = Q.int4_asym_scale_words(*scales)
    pt, st = Q.tile_order("fp8" if fmt == "fp8" else fmt, Q.packed_weight(fmt, codes), scales)
    assert np.array_equal(t["packed"].cpu().numpy().ravel(), pt)
    if fmt == "fp8":
        assert np.array_equal(t["scales"].cpu().numpy(), st)
    else:
        assert np.array_equal(_scale_bytes(t), st)
    assert torch.equal(back["packed"], q["packed"])
    assert torch.equal(back["scales"], q["scales"])


def _layer(fmt, N, K, M, cfg, bias=True):
    W, b, X = synth.linear_case(N, K, M, cfg=cfg, bias=bias)
    q = wq.quantize(fmt, synth.as_torch_bf16(W, DEV))
    return W, b, X, q, wq.repack(q, TILES)


# (M, N, K): every dequant-GEMM launch configuration at shapes whole tiles cover
LINEAR_CASES = [
    (1, 4096, 3072), (2, 1024, 1024),          # one/two rows
    (16, 4096, 3072), (32, 4096, 3072),        # 16/32-row no-split (headline)
    (24, 4096, 6144), (32, 4096, 8192),        # the same over two and three passes of the waves' K steps
    (48, 4096, 3072), (64, 1024, 2048),        # two row blocks, 32- / 16-column tiles
    (100, 4096, 3072),                         # 65-128 rows: 64-column tiles
    (32, 256, 4096), (7, 512, 8192),           # split K + reduction
    (256, 4096, 3072),                         # 64x64 tiles, K groups
    (1536, 2048, 512),                         # 128x128 tiles
    (4096, 4096, 3072),                        # 256x256 tiles
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
def test_linear_same_bits_in_both_layouts(fmt, M, N, K):
    print(f"[case] layouts linear fmt={fmt} M={M} N={N} K={K}", flush=True)
    W, b, X, q, t = _layer(fmt, N, K, M, cfg=800 + M % 89)
    Xd = synth.as_torch_bf16(X, DEV)
    bd = synth.as_torch_bf16(b, DEV)
    Y0 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.linear(Xd, q, bd, out=Y0)
    wq.linear(Xd, t, bd, out=Y1)
    torch.cuda.synchronize()
    assert not torch.isnan(Y0.float()).any()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_tiles_meet_the_oracle_bar(fmt):
    M, N, K = 32, 4096, 3072
    print(f"[case] layouts oracle fmt={fmt}", flush=True)
    W, b, X, q, t = _layer(fmt, N, K, M, cfg=synth.WORKLOADS.get(fmt, {"cfg": 7})["cfg"])
    Y = wq.linear(synth.as_torch_bf16(X, DEV), t, synth.as_torch_bf16(b, DEV))
    torch.cuda.synchronize()
    codes, scales, g = Q.quantize(fmt, W)
    ref = G.linear_fp64(X, Q.dequant(fmt, codes, scales, g), b)
    err = G.rel_frobenius(C.bf16_to_f32(synth.from_torch_bf16(Y)).astype(np.float64), ref)
    print(f"[parity] tiles {fmt}: rel-F {err:.3e}", flush=True)
    assert err <= 1e-2


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_same_bits_in_both_layouts(fmt):
    N, K = 256, 1024
    print(f"[case] layouts dequantize fmt={fmt}", flush=True)
    W = synth.linear_weight(N, K, 901)
    q = wq.quantize(fmt, synth.as_torch_bf16(W, DEV))
    t = wq.repack(q, TILES)
    d0, d1 = wq.dequantize(q), wq.dequantize(t)
    torch.cuda.synchronize()
    assert torch.equal(d0.view(torch.int16), d1.view(torch.int16))
    codes, scales, g = Q.quantize(fmt, W)
    if fmt == "int4_asym":
        return  # its bf16 form is pinned in the parity suite through the rows layout
    assert np.array_equal(synth.from_torch_bf16(d1), Q.dequant_bf16(fmt, codes, scales, g))


@pytest.mark.parametrize("M,N,K", [(1, 4096, 3072), (32, 4096, 3072), (128, 1024, 1024), (256, 4096, 3072),
                                   (1536, 2048, 1024), (4096, 4096, 3072), (7, 256, 8192)])
def test_static_fp8_same_bits_in_both_layouts(M, N, K):
    print(f"[case] layouts static M={M} N={N} K={K}", flush=True)
    W, _, X = synth.linear_case(N, K, M, cfg=910, bias=False)
    Xd = synth.as_torch_bf16(X, DEV)
    scale, _ = wq.calibrate_act_scale([Xd])
    q = wq.quantize("fp8", synth.as_torch_bf16(W, DEV))
    t = wq.repack(q, TILES)
    Y0 = wq.static_fp8_linear(Xd, scale, q["packed"], q["scales"])
    Y1 = wq.static_fp8_linear(Xd, scale, t["packed"], t["scales"], layout=TILES)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(1, 4096, 3072), (32, 4096, 3072), (128, 1024, 3072), (256, 512, 384),
                                   (256, 4096, 3072), (1536, 2048, 1024), (4096, 4096, 3072)])
def test_mx_dynamic_same_bits_in_both_layouts(M, N, K):
    print(f"[case] layouts mx dynamic M={M} N={N} K={K}", flush=True)
    W, b, X, q, t = _layer("mxfp4", N, K, M, cfg=920)
    Xd = synth.as_torch_bf16(X, DEV)
    bd = synth.as_torch_bf16(b, DEV)
    Y0 = wq.mxfp4_dynamic_linear(Xd, q, bd)
    Y1 = wq.mxfp4_dynamic_linear(Xd, t, bd)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))


# seeded shapes over the dequant-GEMM launch regimes, rounded to whole tiles
_rng = np.random.RandomState(20261204)
SWEEP = []
for _i, (_mr, _nr, _kr) in enumerate([((1, 2), (512, 4160), (256, 3072)), ((3, 32), (512, 4160), (256, 3072)),
                                       ((33, 64), (1024, 4416), (256, 2048)), ((65, 128), (3072, 4416), (256, 3072)),
                                       ((1, 64), (32, 640), (3200, 8192)), ((65, 256), (256, 2048), (1024, 3072)),
                                       ((900, 1100), (1536, 2600), (256, 1280))]):
    for _j in range(2):
        SWEEP.append((FMTS[(2 * _i + _j) % len(FMTS)], int(_rng.randint(_mr[0], _mr[1] + 1)),
                      int(_rng.randint(_nr[0], _nr[1] + 1)), int(_rng.randint(_kr[0], _kr[1] + 1)), 940 + 2 * _i + _j))


@pytest.mark.parametrize("fmt,M,N,K,cfg", SWEEP)
def test_tiles_shape_sweep(fmt, M, N, K, cfg):
    nb = 32 if fmt == "mxfp4" else 16
    kb = 64 if fmt == "fp8" else 128
    N, K = max(nb, N // nb * nb), max(kb, K // kb * kb)
    print(f"[case] tiles sweep fmt={fmt} M={M} N={N} K={K}", flush=True)
    W, b, X, q, t = _layer(fmt, N, K, M, cfg=cfg, bias=(cfg % 2 == 0))
    Xd = synth.as_torch_bf16(X, DEV)
    bd = None if b is None else synth.as_torch_bf16(b, DEV)
    Y0, Y1 = wq.linear(Xd, q, bd), wq.linear(Xd, t, bd)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
    codes, scales, g = Q.quantize(fmt, W)
    ref = G.linear_fp64(X, Q.dequant(fmt, codes, scales, g), b)
    err = G.rel_frobenius(C.bf16_to_f32(synth.from_torch_bf16(Y1)).astype(np.float64), ref)
    print(f"[parity] tiles sweep {fmt} M={M} N={N} K={K}: rel-F {err:.3e}", flush=True)
    assert err <= 1e-2
