"""The allocation-free static-FP8 Linear (wq_fp8_static_linear_noalloc, for
callers that cannot allocate device memory) against the entry point it is a
variant of (wq_fp8_static_linear with a caller workspace): the same bits on
consecutive calls through the C ABI, each call smaller than the one before it,
so the library's scratch holds the previous call's larger contents."""

import pytest
import torch

from weight_only_bit_dequant_amd import synth

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(M, N, K, cfg, layout):
    W, b, X = synth.linear_case(N, K, M, cfg=cfg, bias=(cfg % 2 == 0))
    Xd = synth.as_torch_bf16(X, DEV)
    bd = None if b is None else synth.as_torch_bf16(b, DEV)
    scale, _ = wq.calibrate_act_scale([Xd])
    q = wq.quantize("fp8", synth.as_torch_bf16(W, DEV), layout=layout)
    return Xd, bd, scale, q


def test_noalloc_matches_workspace_entry_point():
    # largest first: 4096 x 3072 activations fill 12 MiB of the 16 MiB scratch;
    # then a narrow, deep layer whose plan adds split-K partials; then a small one
    for M, N, K, layout in [(4096, 4096, 3072, wq.LAYOUT_ROWS), (32, 256, 4096, wq.LAYOUT_ROWS),
                            (32, 4096, 3072, wq.LAYOUT_TILES), (7, 512, 1024, wq.LAYOUT_ROWS)]:
        print(f"[case] noalloc M={M} N={N} K={K} layout={layout}", flush=True)
        Xd, bd, scale, q = _case(M, N, K, 970 + M % 13, layout)
        ws = torch.zeros(wq.wq_fp8_static_workspace(M, N, K), dtype=torch.uint8, device=DEV)
        Y0 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        wq.wq_fp8_static_linear(Xd, scale, q["packed"], q["scales"], bd, Y0, ws, layout)
        wq.wq_fp8_static_linear_noalloc(Xd, scale, q["packed"], q["scales"], bd, Y1, layout)
        torch.cuda.synchronize()
        assert not torch.isnan(Y0.float()).any()
        assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))


def test_noalloc_rejects_oversized_problems():
    Xd = torch.zeros((4096, 8192), dtype=torch.bfloat16, device=DEV)
    Wq = torch.zeros((64, 8192), dtype=torch.uint8, device=DEV)
    s = torch.ones(64, dtype=torch.float32, device=DEV)
    Y = torch.empty((4096, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError) as e:
        wq.wq_fp8_static_linear_noalloc(Xd, s[:1], Wq, s, None, Y)
    assert e.value.status == wq.EUNSUPPORTED
