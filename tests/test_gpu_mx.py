"""GPU parity of the MXFP4 dynamic-activation x MXFP4-weight Linear (through
the C ABI) against oracle/mx_dynamic.py on the same seeded inputs.

Bars: activation codes and scales bit-exact; outputs within relative Frobenius
error 1e-2 of the oracle's exact fp64 product of the two MX operands (the MX
products are exact and accumulate in fp32, so the error is the final bf16
rounding).
"""

import numpy as np
import pytest
import torch

from oracle import codecs as C
from oracle import gemm as G
from oracle import mx_dynamic as MX
from oracle import quant as Q
from weight_only_bit_dequant_amd import synth

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_TOL = 1e-2


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


def edge_activations(M, K, seed):
    """Seeded N(0,1) rows plus blocks that hit the rule's corners: an all-zero
    block, negative zeros, a block of bf16 subnormals (e clamps to -127), a
    block whose maximum sits just above 2^-126, ties between E2M1 values and
    values that saturate at 6."""
    x = synth.activations(M, K, seed).copy()
    f = C.bf16_to_f32(x)
    f[0, 0:32] = 0.0
    f[0, 32:64] = -0.0
    if K >= 128:
        f[0, 64:96] = np.float32(2.0 ** -130) * np.arange(32)
        f[0, 96:128] = np.float32(2.0 ** -126) * 1.5
    if M > 1 and K >= 64:
        f[1, 0:8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0]
        f[1, 8:16] = -f[1, 0:8]
        f[1, 32:40] = [6.0, 6.5, 7.9, -8.0, 0.1, -0.1, 3.0, -3.0]
    return C.f32_to_bf16(f)


@pytest.mark.parametrize("M,K", [(1, 3072), (5, 128), (17, 256), (32, 3072), (4096, 3072)])
def test_mx_quantize_act_bit_exact(M, K):
    X = edge_activations(M, K, 500 + M)
    print(f"[case] mx act quant M={M} K={K}", flush=True)
    Xq, Xs = wq.mx_quantize_act(dev_bf16(X))
    torch.cuda.synchronize()
    codes, scales = MX.quantize_act(X)
    assert np.array_equal(host(Xs), scales)
    assert np.array_equal(host(Xq), Q.pack_nibbles(codes))


@pytest.mark.parametrize("M,N,K,bias", [(1, 4096, 3072, True), (17, 256, 512, True), (32, 4096, 3072, True),
                                        (33, 224, 96, False), (64, 512, 1024, True), (100, 128, 256, True),
                                        (200, 256, 160, True), (256, 4096, 3072, True), (4096, 4096, 3072, True),
                                        (300, 512, 1536, False), (1024, 1024, 2560, True),
                                        (3000, 4160, 3200, True), (3000, 4160, 1056, False)])
def test_mx_linear_vs_oracle(M, N, K, bias):
    W, b, X = synth.linear_case(N, K, M, cfg=90 + M)
    b = b if bias else None
    print(f"[case] mx linear M={M} N={N} K={K} bias={bias}", flush=True)
    q = wq.quantize("mxfp4", dev_bf16(W))
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.mxfp4_dynamic_linear(dev_bf16(X), q, dev_bf16(b) if b is not None else None, out=Y)
    torch.cuda.synchronize()
    wc, ws = Q.quantize_mxfp4(W)
    assert np.array_equal(host(q["scales"]), ws)
    # M > 64 runs the tiled kernels: 256x256 tiles straight into LDS when
    # there are >= 192 of them and K % 128 == 0 (ragged M and N tiles and a
    # half-filled last 256-K step at 3000 x 4160 x 3200), else 64x64 or
    # 128x128 tiles through registers (a partial last K step when
    # K % 128 != 0; scale rows preloaded to LDS when K % 512 == 0, else per
    # step, and an odd step count for K = 1536); very large M is checked on a
    # sample of rows
    rows = np.arange(M) if M <= 512 else np.arange(0, M, 61)
    assert_close(Y[torch.as_tensor(rows, device=DEV)], MX.forward(X[rows], wc, ws, b), f"mx M={M} N={N} K={K}")


def test_mx_two_calls_equal_one_call():
    W, b, X = synth.linear_case(4096, 3072, 32, cfg=4)
    q = wq.quantize("mxfp4", dev_bf16(W))
    Xd, bd = dev_bf16(X), dev_bf16(b)
    Y1 = wq.mxfp4_dynamic_linear(Xd, q, bd)
    Xq, Xs = wq.mx_quantize_act(Xd)
    Y2 = torch.empty_like(Y1)
    wq.wq_mx_linear(Xq, Xs, 3072, q["packed"], q["scales"], bd, 4096, Y2)
    Y3 = wq.mxfp4_dynamic_linear(Xd, q, bd)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(Y1.view(torch.int16), Y3.view(torch.int16))


def test_mx_large_tiles_with_unaligned_scales():
    """The 256 x 256 kernel loads scale rows as dwords; with scale arrays that
    are not 4-byte aligned the call takes the register-staged kernel instead.
    Both give the same bits."""
    M, N, K = 2048, 6144, 1024  # 8 x 24 = 192 tiles of 256 x 256
    W, b, X = synth.linear_case(N, K, M, cfg=33)
    print(f"[case] mx large tiles, unaligned scales M={M} N={N} K={K}", flush=True)
    q = wq.quantize("mxfp4", dev_bf16(W))
    Xd, bd = dev_bf16(X), dev_bf16(b)
    Xq, Xs = wq.mx_quantize_act(Xd)
    Y1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    wq.wq_mx_linear(Xq, Xs, K, q["packed"], q["scales"], bd, N, Y1)
    # the same scale bytes at an odd address
    xs_odd = torch.empty(Xs.numel() + 1, dtype=torch.uint8, device=DEV)[1:].view(Xs.shape)
    xs_odd.copy_(Xs)
    ws_odd = torch.empty(q["scales"].numel() + 1, dtype=torch.uint8, device=DEV)[1:].view(q["scales"].shape)
    ws_odd.copy_(q["scales"])
    Y2 = torch.empty_like(Y1)
    wq.wq_mx_linear(Xq, xs_odd, K, q["packed"], ws_odd, bd, N, Y2)
    torch.cuda.synchronize()
    rows = np.arange(0, M, 67)
    wc, ws = Q.quantize_mxfp4(W)
    ref = MX.forward(X[rows], wc, ws, b)
    assert_close(Y1[torch.as_tensor(rows, device=DEV)], ref, "mx 256 tiles")
    assert_close(Y2[torch.as_tensor(rows, device=DEV)], ref, "mx unaligned scales")


@pytest.mark.parametrize("M", [1, 32])
def test_mx_small_m_dword_scales_same_bits(M):
    """Up to 64 rows with K % 128 == 0 the block scales load as dwords (from 9
    rows with K % 512 == 0 the activation rows and scale rows through LDS);
    scale arrays at odd addresses take byte loads straight into registers.
    Both give the same bits."""
    N, K = 4096, 3072
    W, b, X = synth.linear_case(N, K, M, cfg=34 + M)
    print(f"[case] mx small M, dword vs byte scale loads M={M} N={N} K={K}", flush=True)
    q = wq.quantize("mxfp4", dev_bf16(W))
    Xd, bd = dev_bf16(X), dev_bf16(b)
    Xq, Xs = wq.mx_quantize_act(Xd)
    Y1 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    wq.wq_mx_linear(Xq, Xs, K, q["packed"], q["scales"], bd, N, Y1)
    xs_odd = torch.empty(Xs.numel() + 1, dtype=torch.uint8, device=DEV)[1:].view(Xs.shape)
    xs_odd.copy_(Xs)
    ws_odd = torch.empty(q["scales"].numel() + 1, dtype=torch.uint8, device=DEV)[1:].view(q["scales"].shape)
    ws_odd.copy_(q["scales"])
    Y2 = torch.empty_like(Y1)
    wq.wq_mx_linear(Xq, xs_odd, K, q["packed"], ws_odd, bd, N, Y2)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    wc, ws = Q.quantize_mxfp4(W)
    assert_close(Y1, MX.forward(X, wc, ws, b), f"mx small M={M}")


@pytest.mark.parametrize("M,N,K,bias", [
    # the mid-M kernel: more than 64 rows up to 256 tiles of 64 x 64,
    # K % 512 == 0, 1024 <= K <= 4096
    (65, 4096, 1024, True),    # first row count above the small-M kernel; one block per wave, last row tile holds one row
    (200, 1056, 1536, True),   # ragged M and N tiles (N % 64 = 32); 12 blocks: waves 0-3 take two
    (256, 4096, 3072, False),  # 3 blocks per wave, no bias
    (256, 4096, 2560, True),   # 20 blocks: 3 or 2 per wave
    (129, 512, 4096, True),    # the longest K: 4 blocks per wave, 128 KiB of activation rows in LDS
    (1024, 1024, 2048, True),  # 256 tiles; sampled rows
    # the same range outside its limits: the 64 x 64 tiled kernel
    (200, 1056, 1152, True),   # K % 512 != 0
    (130, 256, 9216, True),    # K > 4096
    (768, 4096, 1024, True),   # 768 tiles; sampled rows
])
def test_mx_mid_kernel(M, N, K, bias):
    """The mid-M MX kernel (8 waves split K; activation rows and block scales
    loaded whole into LDS) and, past its limits, the tiled kernel: both weight
    layouts give the same bits, and a repeated call too (fixed-order
    reduction)."""
    W, b, X = synth.linear_case(N, K, M, cfg=600 + M % 50)
    b = b if bias else None
    print(f"[case] mx mid M={M} N={N} K={K} bias={bias}", flush=True)
    q = wq.quantize("mxfp4", dev_bf16(W))
    qt = wq.repack(q, wq.LAYOUT_TILES)
    Xd, bd = dev_bf16(X), dev_bf16(b) if b is not None else None
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.mxfp4_dynamic_linear(Xd, q, bd, out=Y)
    Yt = wq.mxfp4_dynamic_linear(Xd, qt, bd)
    Y2 = wq.mxfp4_dynamic_linear(Xd, q, bd)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yt.view(torch.int16)), "layouts differ"
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), "repeated call differs"
    wc, ws = Q.quantize_mxfp4(W)
    rows = np.arange(M) if M <= 512 else np.arange(0, M, 29)
    assert_close(Y[torch.as_tensor(rows, device=DEV)], MX.forward(X[rows], wc, ws, b), f"mx mid M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [
    (24, 1024, 4096),   # activations through LDS: two passes of 24 steps (4 steps per wave)
    (40, 512, 8192),    # the longest K through LDS: 6 steps per wave, two row blocks
    (16, 256, 512),     # 4 steps: waves 2-11 have none
    (9, 4096, 3072),    # the first row count through LDS
    (8, 4096, 640),     # K % 512 != 0: operands straight into registers, dword scales
    (64, 256, 1152),    # the same with two row tiles per block
    (48, 256, 16384),   # K past the LDS limit: straight into registers
])
def test_mx_small_m_kernels(M, N, K):
    """9 to 64 rows: with K % 512 == 0 and K <= 8192 the workgroup copies its
    activation rows and scale rows into LDS; otherwise (and up to 8 rows) the
    operands load straight into registers.  Both weight layouts give the same
    bits."""
    W, b, X = synth.linear_case(N, K, M, cfg=650 + M)
    print(f"[case] mx small M={M} N={N} K={K}", flush=True)
    q = wq.quantize("mxfp4", dev_bf16(W))
    qt = wq.repack(q, wq.LAYOUT_TILES)
    Xd, bd = dev_bf16(X), dev_bf16(b)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.mxfp4_dynamic_linear(Xd, q, bd, out=Y)
    Yt = wq.mxfp4_dynamic_linear(Xd, qt, bd)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yt.view(torch.int16)), "layouts differ"
    wc, ws = Q.quantize_mxfp4(W)
    assert_close(Y, MX.forward(X, wc, ws, b), f"mx small M={M} N={N} K={K}")
