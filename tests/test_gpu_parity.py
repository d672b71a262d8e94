"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: quantized codes, scales, packed bytes, activation codes and bf16
dequantized weights are bit-exact; GEMM outputs are within relative Frobenius
error 1e-2 of the oracle's fp64 result on the dequantized weight (40 dB by the
static page's sqnr).  Decoding is exact and accumulation is fp32, so the
observed error is the final bf16 rounding (~1e-3); the tests also record it.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs as C
from oracle import gemm as G
from oracle import quant as Q
from oracle import static_fp8 as S
from weight_only_bit_dequant_amd import synth

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_TOL = 1e-2
FMTS = ["int4", "fp8", "nvfp4", "mxfp4", "int4_asym"]


def dev_bf16(bits):
    return synth.as_torch_bf16(bits, DEV)


def host_bits(t):
    return synth.from_torch_bf16(t)


def host(t):
    return t.detach().cpu().numpy()


def gpu_quantize(fmt, W_bits):
    print(f"[case] quantize fmt={fmt} shape={W_bits.shape}", flush=True)
    q = wq.quantize(fmt, dev_bf16(W_bits))
    torch.cuda.synchronize()
    return q


def check_quant_exact(fmt, W_bits, q):
    codes, scales, g = Q.quantize(fmt, W_bits)
    gc = host(q["codes"])
    assert np.array_equal(gc.astype(np.int64), codes.astype(np.int64)), f"{fmt} codes differ"
    if fmt == "int4":
        assert np.array_equal(host(q["scales"].view(torch.int16)).view(np.uint16), scales)
    elif fmt == "int4_asym":
        assert np.array_equal(host(q["scales"]).view(np.uint32), Q.int4_asym_scale_words(*scales))
    elif fmt == "fp8":
        assert np.array_equal(host(q["scales"]).view(np.uint32), scales.view(np.uint32))
    else:
        assert np.array_equal(host(q["scales"]), scales)
    if fmt == "nvfp4":
        assert host(q["global"])[0].view(np.uint32) == np.float32(g).view(np.uint32)
    assert np.array_equal(host(q["packed"]), Q.packed_weight(fmt, codes))
    return codes, scales, g


def run_linear(fmt, W_bits, b_bits, X_bits, q=None):
    if q is None:
        q = gpu_quantize(fmt, W_bits)
    M, K = X_bits.shape
    print(f"[case] linear fmt={fmt} M={M} N={W_bits.shape[0]} K={K}", flush=True)
    X = dev_bf16(X_bits)
    b = dev_bf16(b_bits) if b_bits is not None else None
    Y = torch.full((M, W_bits.shape[0]), float("nan"), dtype=torch.bfloat16, device=DEV)
    wq.linear(X, q, b, out=Y)
    torch.cuda.synchronize()
    return q, Y


def oracle_linear(fmt, W_bits, b_bits, X_bits):
    codes, scales, g = Q.quantize(fmt, W_bits)
    return G.linear_fp64(X_bits, Q.dequant(fmt, codes, scales, g), b_bits)


def assert_close(Y, ref, what):
    y = C.bf16_to_f32(host_bits(Y)).astype(np.float64)
    assert np.isfinite(y).all(), f"{what}: non-finite output (unwritten tile?)"
    err = G.rel_frobenius(y, ref)
    print(f"[parity] {what}: rel-F {err:.3e}  sqnr {G.sqnr_fp64(ref, y):.1f} dB", flush=True)
    assert err <= REL_TOL, f"{what}: rel-F {err}"
    return err


# ------------------------------------------------------------------ quantize / pack / dequant


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(64, 256), (96, 384), (4096, 3072)])
def test_quantize_pack_bit_exact(fmt, shape):
    N, K = shape
    W = synth.linear_weight(N, K, 300 + N)
    q = gpu_quantize(fmt, W)
    check_quant_exact(fmt, W, q)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["zeros", "negzero", "tiny", "wide"])
def test_quantize_edge_weights(fmt, kind):
    W = synth.special_weight(64, 256, 77, kind)
    q = gpu_quantize(fmt, W)
    check_quant_exact(fmt, W, q)


# seeded sweep of quantizer shapes (N and K rounded to each format's rule) and
# weight kinds; WQ_SWEEP_SEED / WQ_SWEEP_PER_REGIME draw another or a larger one
_QPER = int(os.environ.get("WQ_SWEEP_PER_REGIME", "2"))
_qrng = np.random.RandomState(int(os.environ.get("WQ_SWEEP_SEED", "20261206")))
QSWEEP = [(fmt, int(_qrng.randint(1, 3000)), int(_qrng.randint(1, 4500)),
           ["normal", "wide", "negzero", "tiny"][int(_qrng.randint(0, 4))], 320 + 10 * i + j)
          for i, fmt in enumerate(FMTS) for j in range(_QPER)]


@pytest.mark.parametrize("fmt,N,K,kind,seed", QSWEEP)
def test_quantize_sweep_bit_exact(fmt, N, K, kind, seed):
    nb = {"int4": 1, "int4_asym": 1, "fp8": 1, "nvfp4": 16, "mxfp4": 32}[fmt]
    kb = {"int4": 128, "int4_asym": 128, "fp8": 16, "nvfp4": 16, "mxfp4": 32}[fmt]
    N, K = max(nb, N // nb * nb), max(kb, K // kb * kb)
    print(f"[case] quantize sweep fmt={fmt} N={N} K={K} kind={kind}", flush=True)
    W = synth.linear_weight(N, K, seed) if kind == "normal" else synth.special_weight(N, K, seed, kind)
    q = gpu_quantize(fmt, W)
    codes, scales, g = check_quant_exact(fmt, W, q)
    out = wq.dequantize(q)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), Q.dequant_bf16(fmt, codes, scales, g))


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_bf16_bit_exact(fmt):
    W = synth.linear_weight(128, 512, 310)
    q = gpu_quantize(fmt, W)
    codes, scales, g = Q.quantize(fmt, W)
    out = wq.dequantize(q)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), Q.dequant_bf16(fmt, codes, scales, g))


# ------------------------------------------------------------------ fused dequant-GEMM


@pytest.mark.parametrize("fmt", FMTS)
# (2, 4096, 3072): the one- and two-row kernel that loads activations in the
# operand layout directly (256 workgroups, no split)
@pytest.mark.parametrize("M,N,K", [(1, 128, 256), (2, 4096, 3072), (17, 256, 512), (32, 192, 384), (33, 320, 768),
                                   (64, 256, 1024), (100, 128, 256)])
def test_linear_small_shapes(fmt, M, N, K):
    W, b, X = synth.linear_case(N, K, M, cfg=20 + M)
    _, Y = run_linear(fmt, W, b, X)
    assert_close(Y, oracle_linear(fmt, W, b, X), f"{fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt,N", [("int4", 4100), ("fp8", 4100), ("nvfp4", 4112), ("mxfp4", 4128), ("int4_asym", 4100)])
@pytest.mark.parametrize("M", [40, 64])
def test_linear_two_row_blocks_wide(fmt, N, M):
    # 33..64 rows on a wide layer: two row blocks of 32-column workgroups
    # (256 and more of them), with a column tail inside the last tile
    W, b, X = synth.linear_case(N, 512, M, cfg=36 + M)
    _, Y = run_linear(fmt, W, b, X)
    assert_close(Y, oracle_linear(fmt, W, b, X), f"{fmt} M={M} N={N}")


@pytest.mark.parametrize("fmt,N", [("int4", 4100), ("fp8", 4100), ("nvfp4", 4112), ("mxfp4", 4128), ("int4_asym", 4100)])
@pytest.mark.parametrize("M", [65, 100, 128])
def test_linear_wide_64_column_tiles(fmt, N, M):
    # 65..128 rows on a wide layer: three or four row blocks of 64-column
    # workgroups of 8 waves, with a column tail inside the last tile
    W, b, X = synth.linear_case(N, 768, M, cfg=40 + M)
    _, Y = run_linear(fmt, W, b, X)
    assert_close(Y, oracle_linear(fmt, W, b, X), f"{fmt} M={M} N={N}")


@pytest.mark.parametrize("fmt,N", [("int4", 200), ("fp8", 200), ("nvfp4", 208), ("mxfp4", 224), ("int4_asym", 200)])
@pytest.mark.parametrize("K", [256, 4096])
@pytest.mark.parametrize("M", [2, 5, 40])
def test_linear_ragged_n(fmt, N, K, M):
    # A narrow layer with a column tail.  K = 256 runs the no-split tiles (16
    # columns per workgroup: INT4 and FP8 at N = 200 end in a half tile); K =
    # 4096 splits K across workgroups of 64 columns and sums them in the
    # reduction kernel, where every N here ends in a partial tile (N % 64 =
    # 8, 16, 32).  M = 2 and 5 take one row block, M = 40 two.
    W, b, X = synth.linear_case(N, K, M, cfg=33)
    _, Y = run_linear(fmt, W, b, X)
    assert_close(Y, oracle_linear(fmt, W, b, X), f"{fmt} ragged N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_no_bias(fmt):
    W, _, X = synth.linear_case(128, 256, 8, cfg=34, bias=False)
    _, Y = run_linear(fmt, W, None, X)
    assert_close(Y, oracle_linear(fmt, W, None, X), f"{fmt} no bias")


@pytest.mark.parametrize("fmt", FMTS)
def test_linear_full_size_m32(fmt):
    """The benchmark workload: nn.Linear(3072, 4096), bf16, bias, M=32, in the
    launch configuration the benchmark times."""
    cfg = synth.WORKLOADS[fmt]["cfg"]
    W, b, X = synth.linear_case(4096, 3072, 32, cfg=cfg)
    q, Y = run_linear(fmt, W, b, X)
    check_quant_exact(fmt, W, q)
    assert_close(Y, oracle_linear(fmt, W, b, X), f"{fmt} 4096x3072 M=32")
    # run twice: fixed-order reduction gives identical bits
    Y2 = wq.linear(dev_bf16(X), q, dev_bf16(b))
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))


@pytest.mark.parametrize("M", [1, 256, 4096])
def test_linear_mxfp4_m_sweep(M):
    W, b, X = synth.linear_case(4096, 3072, M, cfg=4)
    q, Y = run_linear("mxfp4", W, b, X)
    if M <= 256:
        assert_close(Y, oracle_linear("mxfp4", W, b, X), f"mxfp4 M={M}")
    else:
        # oracle on a sample of rows (every row is computed independently)
        rows = np.arange(0, M, 97)
        ref = oracle_linear("mxfp4", W, b, X[rows])
        assert_close(Y[torch.as_tensor(rows, device=DEV)], ref, f"mxfp4 M={M} sampled rows")


# (M, N, K) -> tile shape / K groups chosen by the plan (64x64 tiles split K
# over four groups of 2 waves for the 4-bit formats, two groups of 4 for FP8):
#   64x64 tiles in K groups (34 steps; 33 steps: the last group's range ends
#   early), 64x64 in K groups, 128x64 in 2 groups, 64x128 in 2 groups (ragged
#   N), 64x64 with ragged M; the last two take 256x256 tiles in every format
#   (ragged M and N tiles; the last with a partial final K step)
TILED_CASES = [(256, 1024, 2176), (256, 1024, 2112), (640, 2048, 1152), (384, 4096, 1024), (6144, 192, 1024),
               (200, 1024, 2048), (3000, 4000, 1024), (2900, 4160, 1120)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", TILED_CASES)
def test_linear_tiled_k_groups(fmt, M, N, K):
    if fmt in ("int4", "int4_asym") and K % 128:
        pytest.skip("INT4 groups need K % 128 == 0")
    W, b, X = synth.linear_case(N, K, M, cfg=80 + M % 7)
    _, Y = run_linear(fmt, W, b, X)
    rows = np.arange(M) if M <= 1024 else np.arange(0, M, 37)
    ref = oracle_linear(fmt, W, b, X[rows])
    assert_close(Y[torch.as_tensor(rows, device=DEV)], ref, f"{fmt} tiled M={M} N={N} K={K}")


def test_linear_dense_bf16():
    W, b, X = synth.linear_case(4096, 3072, 32, cfg=6)
    print("[case] dense bf16 linear", flush=True)
    Y = wq.linear(dev_bf16(X), wq.dense(dev_bf16(W)), dev_bf16(b))
    torch.cuda.synchronize()
    ref = G.linear_fp64(X, C.bf16_to_f32(W).astype(np.float64), b)
    assert_close(Y, ref, "bf16 dense M=32")


def test_linear_empty_calls():
    W, b, X = synth.linear_case(64, 256, 4, cfg=35)
    q = gpu_quantize("int4", W)
    Y = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    wq.linear(dev_bf16(X)[:0], q, None, out=Y)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ static FP8


def test_static_act_quant_and_calibration_bit_exact():
    X = synth.activations(64, 3072, 400)
    print("[case] static act quant", flush=True)
    scale, amax = wq.calibrate_act_scale([dev_bf16(X)])
    Xq = torch.empty((64, 3072), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_quantize_act(dev_bf16(X), scale, Xq)
    torch.cuda.synchronize()
    a_ref = S.absmax(X)
    s_ref = S.scale_from_amax(a_ref)
    assert host(amax)[0] == a_ref
    assert host(scale)[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
    assert np.array_equal(host(Xq), S.quantize_act(X, s_ref))
    # ragged element count (M*K not a multiple of 8)
    X2 = synth.activations(3, 40, 401)
    Xq2 = torch.empty((3, 40), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_quantize_act(dev_bf16(X2), scale, Xq2)
    torch.cuda.synchronize()
    assert np.array_equal(host(Xq2), S.quantize_act(X2, s_ref))


@pytest.mark.parametrize("scale", [1.0, 0.0, 3.0, 0.0123, 448.0 / 3.0e4, 2.0 ** -10, 7.5e-5, 1.7e3])
def test_static_act_quant_every_bf16(scale):
    """Every non-NaN bf16 value (infinities, zeros, subnormals included)
    through the static activation Q at several scales: the E4M3 codes equal
    the oracle's bit for bit.  The quotients x / s cover the E4M3 subnormal
    range, rounding ties and saturation.  The element count is ragged
    (65282 = 8 * 8160 + 2)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    nan = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)
    X = bits[~nan].reshape(1, -1)
    print(f"[case] static act quant every bf16, scale {scale}", flush=True)
    t_s = torch.tensor([scale], dtype=torch.float32, device=DEV)
    Xq = torch.empty(X.shape, dtype=torch.uint8, device=DEV)
    wq.wq_fp8_quantize_act(dev_bf16(X), t_s, Xq)
    torch.cuda.synchronize()
    assert np.array_equal(host(Xq), S.quantize_act(X, np.float32(scale)))


def test_static_act_quant_beyond_one_grid_pass():
    """An activation tensor with more 8-element chunks than one capped grid
    covers (2^24 chunks), plus a ragged tail: the threads stride over the
    rest.  Checked on slices around the first pass's end and at both ends
    (the Q is elementwise, so the oracle runs on each slice alone)."""
    n = (1 << 27) + (1 << 20) + 13
    print(f"[case] static act quant numel={n}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(404)
    x = (torch.randn(1, n, generator=gen, device=DEV) * 3.0).to(torch.bfloat16)
    t_s = torch.tensor([0.0123], dtype=torch.float32, device=DEV)
    xq = torch.empty((1, n), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_quantize_act(x, t_s, xq)
    torch.cuda.synchronize()
    for a, b in [(0, 1 << 16), ((1 << 27) - (1 << 16), (1 << 27) + (1 << 16)), (n - (1 << 16) - 13, n)]:
        xs = host_bits(x[:, a:b].contiguous())
        assert np.array_equal(host(xq[:, a:b]), S.quantize_act(xs, np.float32(0.0123))), (a, b)


def _gpu_static_layer(x_dev, act_scale, Wq, w_scale):
    return wq.static_fp8_linear(x_dev, act_scale, Wq, w_scale)


def test_static_two_layer_mlp():
    """The static page's model: Linear(256, 512) -> Linear(512, 128), no bias,
    calibrated on 10 batches; GPU vs oracle per layer and end to end."""
    weights = synth.mlp_weights()
    batches = synth.calibration_batches(32, 256)
    scales_ref, amax_ref = S.calibrate(batches, weights)
    print("[case] static MLP calibration", flush=True)
    # GPU calibration: absmax observers over the float model (dense bf16 linear)
    Wd = [dev_bf16(w) for w in weights]
    amax1 = torch.zeros(1, dtype=torch.float32, device=DEV)
    amax2 = torch.zeros(1, dtype=torch.float32, device=DEV)
    for xb in batches:
        x = dev_bf16(xb)
        wq.wq_absmax(x, amax1)
        h = wq.linear(x, wq.dense(Wd[0]))
        wq.wq_absmax(h, amax2)
    s1 = torch.empty(1, dtype=torch.float32, device=DEV)
    s2 = torch.empty(1, dtype=torch.float32, device=DEV)
    wq.wq_fp8_scale(amax1, s1)
    wq.wq_fp8_scale(amax2, s2)
    torch.cuda.synchronize()
    assert host(amax1)[0] == amax_ref[0]
    # layer-2 amax comes from bf16 GEMM outputs: fp32 accumulation may move a
    # bf16 rounding by one unit relative to the fp64 oracle
    assert abs(float(host(amax2)[0]) - float(amax_ref[1])) <= float(amax_ref[1]) * 2.0 ** -7
    qd = [wq.quantize("fp8", w) for w in Wd]
    qref = S.quantize_model(weights)
    for qq, (c, s) in zip(qd, qref):
        assert np.array_equal(host(qq["codes"]), c)
        assert np.array_equal(host(qq["scales"]).view(np.uint32), s.view(np.uint32))
    x = synth.activations(32, 256, synth.SEED_X + 5)
    h = _gpu_static_layer(dev_bf16(x), s1, qd[0]["codes"], qd[0]["scales"])
    y = _gpu_static_layer(h, s2, qd[1]["codes"], qd[1]["scales"])
    torch.cuda.synchronize()
    y_ref, outs = S.quant_forward(x, [np.float32(host(s1)[0]), np.float32(host(s2)[0])], qref)
    # per-layer parity with the oracle's own layer input
    h_ref = S.static_linear_fp64(S.quantize_act(x, host(s1)[0]), host(s1)[0], *qref[0])
    assert_close(h, h_ref, "static layer 1")
    assert_close(y, y_ref, "static MLP end to end")
    _, fp_out = S.float_forward(x, weights)
    v = G.sqnr(C.bf16_to_f32(fp_out), C.bf16_to_f32(host_bits(y)))
    print(f"[parity] static MLP eager SQNR vs float model: {v:.2f} dB (oracle "
          f"{G.sqnr(C.bf16_to_f32(fp_out), C.bf16_to_f32(outs[-1])):.2f} dB)", flush=True)


@pytest.mark.parametrize("M", [32, 4096])
def test_static_large_layer(M):
    """3072 -> 4096 static-FP8 layer, calibrated on 10 seeded [32, 3072] batches."""
    W = synth.linear_weight(4096, 3072, synth.SEED_W + 5)
    batches = [synth.activations(32, 3072, synth.SEED_CAL + 100 + i) for i in range(10)]
    print(f"[case] static large M={M}", flush=True)
    scale, amax = wq.calibrate_act_scale([dev_bf16(b) for b in batches])
    s_ref = S.scale_from_amax(max(S.absmax(b) for b in batches))
    assert host(scale)[0].view(np.uint32) == np.float32(s_ref).view(np.uint32)
    q = wq.quantize("fp8", dev_bf16(W))
    X = synth.activations(M, 3072, synth.SEED_X + 5)
    Y = wq.static_fp8_linear(dev_bf16(X), scale, q["codes"], q["scales"])
    torch.cuda.synchronize()
    wq_ref, ws_ref = Q.quantize_fp8_row(W)
    rows = np.arange(M) if M <= 64 else np.arange(0, M, 61)
    ref = S.static_linear_fp64(S.quantize_act(X[rows], s_ref), s_ref, wq_ref, ws_ref)
    assert_close(Y[torch.as_tensor(rows, device=DEV)], ref, f"static 3072->4096 M={M}")


@pytest.mark.parametrize("M,N,K,bias", [(32, 4096, 3072, False), (2, 4096, 3072, True), (17, 200, 512, True),
                                        (64, 256, 1024, True), (48, 4112, 1024, True), (256, 4096, 3072, False),
                                        (640, 2048, 1152, True)])
def test_fp8_linear_on_prequantized_activations(M, N, K, bias):
    """wq_fp8_quantize_act then wq_fp8_linear equals wq_fp8_static_linear bit
    for bit (same kernels) and the oracle's fp64 DQ-GEMM within the bar."""
    W, b, X = synth.linear_case(N, K, M, cfg=70 + M)
    b = b if bias else None
    cal = synth.activations(32, K, synth.SEED_CAL + 300)
    print(f"[case] fp8_linear M={M} N={N} K={K} bias={bias}", flush=True)
    scale, _ = wq.calibrate_act_scale([dev_bf16(cal)])
    q = wq.quantize("fp8", dev_bf16(W))
    Xd = dev_bf16(X)
    bd = dev_bf16(b) if b is not None else None
    Xq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_quantize_act(Xd, scale, Xq)
    Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(1, wq.wq_fp8_linear_workspace(M, N, K)), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_linear(Xq, scale, q["codes"], q["scales"], bd, Y1, ws)
    Y2 = wq.static_fp8_linear(Xd, scale, q["codes"], q["scales"], bd)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    s_ref = S.scale_from_amax(S.absmax(cal))
    wq_ref, ws_ref = Q.quantize_fp8_row(W)
    xq_ref = S.quantize_act(X, s_ref)
    assert np.array_equal(host(Xq), xq_ref)
    assert_close(Y1, S.static_linear_fp64(xq_ref, s_ref, wq_ref, ws_ref, b), f"fp8_linear M={M} N={N}")


@pytest.mark.parametrize("M,N,K,bias", [(3000, 4160, 1040, True), (520, 6000, 208, True), (1000, 1000, 1104, False)])
def test_fp8_tiled_ragged(M, N, K, bias):
    """Static-FP8 GEMM in its three tiled forms (256 x 256, 128 x 128 and
    64 x 64 tiles, chosen by the tile count) with ragged M and N tiles and a
    partial last K step; sampled rows against the oracle."""
    W, b, X = synth.linear_case(N, K, M, cfg=90 + K % 7)
    b = b if bias else None
    print(f"[case] fp8 tiled ragged M={M} N={N} K={K} bias={bias}", flush=True)
    scale, _ = wq.calibrate_act_scale([dev_bf16(X[:64])])
    q = wq.quantize("fp8", dev_bf16(W))
    Xq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_quantize_act(dev_bf16(X), scale, Xq)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(1, wq.wq_fp8_linear_workspace(M, N, K)), dtype=torch.uint8, device=DEV)
    wq.wq_fp8_linear(Xq, scale, q["codes"], q["scales"], dev_bf16(b) if b is not None else None, Y, ws)
    torch.cuda.synchronize()
    s_ref = S.scale_from_amax(S.absmax(X[:64]))
    wq_ref, ws_ref = Q.quantize_fp8_row(W)
    rows = np.unique(np.concatenate([np.arange(0, M, 37), [M - 1]]))
    ref = S.static_linear_fp64(S.quantize_act(X[rows], s_ref), s_ref, wq_ref, ws_ref, b)
    assert_close(Y[torch.as_tensor(rows, device=DEV)], ref, f"fp8 tiled M={M} N={N} K={K}")


@pytest.mark.parametrize("nbytes", [16, 1040, 16384 + 48, 4096 * 1536])
def test_read_stream_xor(nbytes):
    """The measurement stream reads every byte: each block's XOR equals the host's."""
    rng = np.random.default_rng(nbytes)
    host_words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    print(f"[case] read_stream bytes={nbytes}", flush=True)
    buf = torch.from_numpy(host_words.view(np.int32)).to(DEV)
    nw = wq.wq_read_stream_words(nbytes)
    assert nw == -(-nbytes // 16384)
    sink = torch.full((nw + 1,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    wq.wq_read_stream(buf, sink)
    torch.cuda.synchronize()
    got = host(sink).view(np.uint32)
    for blk in range(nw):
        assert got[blk] == np.bitwise_xor.reduce(host_words[blk * 4096:(blk + 1) * 4096]), blk
    assert got[nw] == 0x5A5A5A5A  # nothing written past the last block


def test_workspace_reuse_across_plans():
    """Calls with different launch plans (K split across workgroups or not)
    share one cached workspace and run back to back."""
    cases = [(32, 4096, 3072), (64, 256, 4096), (16, 1024, 6144), (64, 256, 4096), (32, 4096, 3072)]
    for i, (M, N, K) in enumerate(cases):
        W, b, X = synth.linear_case(N, K, M, cfg=60 + i)
        _, Y = run_linear("int4", W, b, X)
        assert_close(Y, oracle_linear("int4", W, b, X), f"reuse {i} M={M} N={N} K={K}")
