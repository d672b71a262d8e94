"""The C-ABI library loads, exports every symbol include/wq.h declares, and
rejects bad arguments on the host before touching HIP (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")

if not os.path.exists(wq.LIB_PATH):  # pragma: no cover
    pytest.skip("libwq.so not built", allow_module_level=True)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = wq.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    L = wq.lib()
    assert L.wq_abi_version() == 2
    assert L.wq_status_str(0) == b"WQ_OK"
    assert L.wq_status_str(2) == b"WQ_ESHAPE"
    assert L.wq_status_str(99) == b"WQ_UNKNOWN"


def test_layout_sizes():
    assert wq.wq_layout("int4", 4096, 3072) == (4096 * 3072, 4096 * 1536, 4096 * 24 * 2, 0)
    assert wq.wq_layout("fp8", 4096, 3072) == (4096 * 3072, 4096 * 3072, 4096 * 4, 0)
    assert wq.wq_layout("nvfp4", 4096, 3072) == (4096 * 3072, 4096 * 1536, 4096 * 192, 4)
    assert wq.wq_layout("mxfp4", 4096, 3072) == (4096 * 3072, 4096 * 1536, 4096 * 96, 0)
    assert wq.wq_layout("bf16", 8, 16) == (256, 256, 0, 0)
    assert wq.wq_layout("int4_asym", 4096, 3072) == (4096 * 3072, 4096 * 1536, 4096 * 24 * 4, 0)


@pytest.mark.parametrize("fmt,N,K", [("int4", 64, 100), ("nvfp4", 40, 64), ("nvfp4", 64, 40), ("mxfp4", 48, 64),
                                     ("mxfp4", 64, 48), ("int4_asym", 64, 192)])
def test_shape_rules(fmt, N, K):
    with pytest.raises(ValueError) as e:
        wq.wq_layout(fmt, N, K)
    assert e.value.status == wq.ESHAPE


def _call_linear(fmt=1, X=16, M=32, K=256, W=32, S=48, G=None, B=None, N=64, Y=64, ws=None, wsb=0, layout=0):
    L = wq.lib()
    v = ctypes.c_void_p
    return L.wq_linear(fmt, v(X), M, K, v(W), layout, v(S), v(G), v(B), N, v(Y), v(ws), wsb, None)


def test_linear_host_validation():
    # pointers below are fake; every call fails validation before any HIP call
    assert _call_linear(fmt=9) == wq.EINVAL
    assert _call_linear(M=-1) == wq.EINVAL
    assert _call_linear(K=100) == wq.ESHAPE  # INT4 group
    assert _call_linear(fmt=3, N=40, G=64) == wq.ESHAPE  # NVFP4 %16
    assert _call_linear(fmt=4, K=48) == wq.ESHAPE  # MXFP4 %32
    assert _call_linear(fmt=2, K=24) == wq.EUNSUPPORTED  # FP8 kernel needs K % 16
    assert _call_linear(fmt=3, K=48, N=64, G=64) == wq.EUNSUPPORTED  # NVFP4 kernel needs K % 32
    assert _call_linear(X=None) == wq.EINVAL
    assert _call_linear(S=None) == wq.EINVAL
    assert _call_linear(fmt=3, G=None) == wq.EINVAL  # NVFP4 needs its global scale
    assert _call_linear(fmt=1, G=64) == wq.EINVAL  # global scale only for NVFP4
    assert _call_linear(X=24) == wq.EALIGN
    assert _call_linear(Y=8) == wq.EALIGN
    # M = 0 and N = 0 are empty calls (nothing launched)
    assert _call_linear(M=0) == wq.OK
    assert _call_linear(N=0) == wq.OK
    # split-K needs a workspace: a narrow layer (256 columns) splits K
    need = wq.wq_linear_workspace("int4", 32, 256, 4096)
    assert need > 0
    assert _call_linear(M=32, K=4096, N=256, ws=None) == wq.EWORKSPACE
    assert _call_linear(M=32, K=4096, N=256, ws=64, wsb=need - 1) == wq.EWORKSPACE
    assert b"workspace" in wq.lib().wq_last_error()


def test_quantize_pack_dequant_validation():
    L = wq.lib()
    v = ctypes.c_void_p
    assert L.wq_quantize(0, v(16), 64, 64, v(16), v(16), None, None) == wq.EINVAL  # BF16 has no quantizer
    assert L.wq_quantize(3, v(16), 64, 64, v(16), v(16), None, None) == wq.EINVAL  # NVFP4 needs global
    assert L.wq_quantize(1, v(16), 64, 64, v(16), v(16), None, None) == wq.ESHAPE
    assert L.wq_quantize(4, v(8), 64, 64, v(16), v(16), None, None) == wq.EALIGN
    assert L.wq_quantize(2, None, 64, 64, v(16), v(16), None, None) == wq.EINVAL
    assert L.wq_quantize(2, None, 0, 64, None, None, None, None) == wq.OK
    assert L.wq_pack(0, v(16), 64, 64, v(16), None) == wq.EINVAL
    assert L.wq_pack(4, v(16), 64, 40, v(16), None) == wq.ESHAPE
    assert L.wq_dequantize(3, v(16), 0, v(16), None, 64, 64, v(16), None) == wq.EINVAL
    assert L.wq_dequantize(2, v(16), 0, v(16), None, 64, 12, v(16), None) == wq.EUNSUPPORTED
    assert L.wq_dequantize(4, v(16), 1, v(16), None, 64, 96, v(16), None) == wq.EUNSUPPORTED  # tiles: K % 128
    assert L.wq_fp8_quantize_act(v(16), 4, 16, None, v(16), None) == wq.EINVAL
    assert L.wq_fp8_quantize_act(v(16), 1 << 22, 1 << 21, v(16), v(16), None) == wq.EUNSUPPORTED  # 2^43 elements
    assert L.wq_fp8_static_linear(v(16), 4, 24, v(16), v(16), 0, v(16), None, 16, v(16), v(16), 1 << 20,
                                  None) == wq.EUNSUPPORTED
    assert L.wq_fp8_static_linear(v(16), 4, 32, v(16), v(16), 0, v(16), None, 16, v(16), None, 0,
                                  None) == wq.EWORKSPACE
    assert L.wq_absmax(None, 10, v(16), None) == wq.EINVAL
    assert L.wq_absmax(None, 0, None, None) == wq.OK
    # FP8 GEMM on pre-quantized activations
    assert L.wq_fp8_linear(v(16), 4, 24, v(16), v(16), 0, v(16), None, 16, v(16), None, 0, None) == wq.EUNSUPPORTED
    assert L.wq_fp8_linear(v(16), 4, 32, None, v(16), 0, v(16), None, 16, v(16), None, 0, None) == wq.EINVAL
    assert L.wq_fp8_linear(v(8), 4, 32, v(16), v(16), 0, v(16), None, 16, v(16), None, 0, None) == wq.EALIGN
    assert L.wq_fp8_linear(v(16), 0, 32, v(16), v(16), 0, v(16), None, 16, v(16), None, 0, None) == wq.OK
    assert L.wq_fp8_linear(v(16), 32, 4096, v(16), v(16), 0, v(16), None, 256, v(16), None, 0,
                           None) == wq.EWORKSPACE  # narrow layer: split K
    # MXFP4 dynamic-activation path
    assert L.wq_mx_quantize_act(v(16), 4, 48, v(16), v(16), None) == wq.ESHAPE
    assert L.wq_mx_quantize_act(v(16), 4, 64, None, v(16), None) == wq.EINVAL
    assert L.wq_mx_quantize_act(v(8), 4, 64, v(16), v(16), None) == wq.EALIGN
    assert L.wq_mx_quantize_act(None, 0, 64, None, None, None) == wq.OK
    assert L.wq_mx_linear(v(16), v(16), 4, 64, v(16), 0, v(16), None, 48, v(16), None) == wq.ESHAPE  # N % 32
    assert L.wq_mx_linear(v(16), v(16), 4, 48, v(16), 0, v(16), None, 64, v(16), None) == wq.ESHAPE  # K % 32
    assert L.wq_mx_linear(v(16), None, 4, 64, v(16), 0, v(16), None, 64, v(16), None) == wq.EINVAL
    assert L.wq_mx_linear(v(16), v(16), 4, 64, v(16), 0, v(16), None, 64, v(24), None) == wq.EALIGN
    need = wq.wq_mxfp4_dynamic_workspace(32, 3072)
    assert need >= 32 * 1536 + 32 * 96
    assert L.wq_mxfp4_dynamic_linear(v(16), 32, 3072, v(16), 0, v(16), None, 4096, v(16), v(16), need - 1,
                                     None) == wq.EWORKSPACE
    assert L.wq_mxfp4_dynamic_linear(v(16), 0, 3072, v(16), 0, v(16), None, 4096, v(16), None, 0, None) == wq.OK
    assert L.wq_mxfp4_dynamic_linear(v(16), 4, 96, v(16), 1, v(16), None, 64, v(16), v(16), 1 << 20,
                                     None) == wq.EUNSUPPORTED  # tiles need K % 128
    # fused static MLP
    mlp = lambda M=32, K1=256, N1=512, N2=128, X=16: L.wq_fp8_static_mlp2(
        v(X), M, K1, v(16), v(16), v(16), None, N1, v(16), v(16), v(16), None, N2, v(16), None)
    assert mlp(K1=24) == wq.EUNSUPPORTED
    assert mlp(N1=40) == wq.EUNSUPPORTED
    assert mlp(K1=8192, N1=4096) == wq.EUNSUPPORTED  # 16 rows exceed the LDS
    assert mlp(X=8) == wq.EALIGN
    assert mlp(M=1 << 20, K1=1024, N1=256, N2=64) == wq.EUNSUPPORTED  # activation buffer of 2^31 bytes
    assert mlp(M=0) == wq.OK
    # read-only stream (measurement aid)
    assert L.wq_read_stream(v(16), 0, None, None) == wq.OK
    assert L.wq_read_stream(None, 64, v(16), None) == wq.EINVAL
    assert L.wq_read_stream(v(8), 64, v(16), None) == wq.EALIGN
    assert L.wq_read_stream(v(16), 40, v(16), None) == wq.EUNSUPPORTED


def test_workspace_plans_are_consistent():
    # empty or invalid problems need no workspace; the static path adds the
    # quantized-activation buffer (M*K rounded to 256) to the GEMM's
    assert wq.wq_linear_workspace("int4", 0, 4096, 3072) == 0
    assert wq.wq_linear_workspace(9, 32, 4096, 3072) == 0
    M, N, K = 32, 4096, 3072
    gemm = wq.wq_linear_workspace("fp8", M, N, K)
    assert wq.wq_fp8_static_workspace(M, N, K) >= gemm + M * K
    assert wq.wq_fp8_linear_workspace(M, N, K) == 0
    assert wq.wq_fp8_linear_workspace(32, 256, 4096) > 0
    assert wq.wq_fp8_static_workspace(32, 256, 4096) >= wq.wq_fp8_linear_workspace(32, 256, 4096) + 32 * 4096
    # wide layers have enough workgroups without K splits
    assert wq.wq_linear_workspace("mxfp4", 4096, 4096, 3072) == 0
    assert wq.wq_linear_workspace("int4", 32, 4096, 3072) == 0


def _launch_attempts():
    """Launch attempts so far in the sanitizer host-check build (None in the
    real library, where a launch without a GPU fails with WQ_EHIP instead)."""
    f = getattr(wq.lib(), "wq_hostcheck_launches", None)
    if f is None:
        return None
    f.restype = ctypes.c_long
    return f()


def test_static_linear_validates_both_launches_first():
    """The static-FP8 Linear runs two kernels (activation Q, then the FP8
    GEMM); a GEMM-only limit (K of 2^22 or more) must be rejected before the
    first one is enqueued: the status is WQ_EUNSUPPORTED, not the WQ_EHIP a
    launch attempt gives without a GPU, and no launch was attempted."""
    L = wq.lib()
    v = ctypes.c_void_p
    K = 1 << 22
    need = wq.wq_fp8_static_workspace(1, 16, K)
    before = _launch_attempts()
    assert L.wq_fp8_static_linear(v(16), 1, K, v(16), v(16), 0, v(16), None, 16, v(16), v(256), need, None) == \
        wq.EUNSUPPORTED
    assert b"2^22" in L.wq_last_error()
    assert _launch_attempts() == before


def test_layout_validation():
    """Tile order (layout 1) needs whole 16-row x 64-byte tiles; BF16 has only
    the rows layout; unknown layouts are rejected -- all before any launch."""
    assert _call_linear(layout=2) == wq.EINVAL
    assert _call_linear(fmt=0, K=256, S=None, layout=1) == wq.EUNSUPPORTED  # BF16
    assert _call_linear(fmt=1, N=40, layout=1) == wq.EUNSUPPORTED  # N % 16
    assert _call_linear(fmt=4, K=96, layout=1) == wq.EUNSUPPORTED  # 4-bit: K % 128
    assert _call_linear(fmt=2, K=96, layout=1) == wq.EUNSUPPORTED  # FP8: K % 64
    assert _call_linear(fmt=2, M=0, K=128, layout=1) == wq.OK  # empty call
    L = wq.lib()
    v = ctypes.c_void_p
    assert L.wq_repack(0, 64, 256, 0, v(16), v(16), 1, v(32), v(32), None) == wq.EINVAL  # BF16
    assert L.wq_repack(4, 64, 256, 0, v(16), v(16), 3, v(32), v(32), None) == wq.EINVAL  # layout 3
    assert L.wq_repack(4, 48, 256, 0, v(16), v(16), 1, v(32), v(32), None) == wq.ESHAPE  # MXFP4 N % 32
    assert L.wq_repack(1, 40, 256, 0, v(16), v(16), 1, v(32), v(32), None) == wq.EUNSUPPORTED  # tiles: N % 16
    assert L.wq_repack(1, 64, 256, 0, v(16), v(16), 1, v(16), v(32), None) == wq.EINVAL  # in place
    assert L.wq_repack(1, 64, 256, 0, None, v(16), 1, v(32), v(32), None) == wq.EINVAL
    assert L.wq_repack(1, 64, 256, 0, v(16), v(8), 1, v(32), v(48), None) == wq.EALIGN
    assert L.wq_repack(1, 0, 256, 0, None, None, 1, None, None, None) == wq.OK
    assert L.wq_fp8_linear(v(16), 4, 96, v(16), v(16), 1, v(16), None, 16, v(16), None, 0, None) == wq.EUNSUPPORTED
    assert L.wq_mx_linear(v(16), v(16), 4, 96, v(16), 1, v(16), None, 64, v(16), None) == wq.EUNSUPPORTED


def test_noalloc_static_linear_limits():
    """The allocation-free static-FP8 Linear rejects problems whose scratch
    would exceed its fixed 16 MiB before touching HIP."""
    L = wq.lib()
    v = ctypes.c_void_p
    before = _launch_attempts()
    # M * K = 32 Mi activations: E4M3 copy alone is 32 MiB
    assert L.wq_fp8_static_linear_noalloc(v(16), 4096, 8192, v(16), v(16), 0, v(16), None, 4096, v(16),
                                          None) == wq.EUNSUPPORTED
    assert b"16777216" in L.wq_last_error()
    assert L.wq_fp8_static_linear_noalloc(v(16), 4, 24, v(16), v(16), 0, v(16), None, 16, v(16), None) == \
        wq.EUNSUPPORTED  # K % 16
    assert L.wq_fp8_static_linear_noalloc(v(16), 0, 32, v(16), v(16), 0, v(16), None, 16, v(16), None) == wq.OK
    assert L.wq_fp8_static_linear_noalloc(v(16), -1, 32, v(16), v(16), 0, v(16), None, 16, v(16), None) == wq.EINVAL
    assert _launch_attempts() == before


def test_two_kernel_form_validation():
    L = wq.lib()
    v = ctypes.c_void_p
    need = wq.wq_linear_dq_gemm_workspace("mxfp4", 32, 4096, 3072)
    assert need >= 4096 * 3072 * 2
    assert wq.wq_linear_dq_gemm_workspace("bf16", 32, 64, 64) == 0
    call = lambda fmt=4, M=32, K=3072, N=4096, ws=256, wsb=need, layout=0, X=16: L.wq_linear_dq_gemm(
        fmt, v(X), M, K, v(16), layout, v(16), None, None, N, v(16), v(ws), wsb, None)
    assert call(fmt=0) == wq.EINVAL  # nothing to dequantize
    assert call(K=48) == wq.ESHAPE
    assert call(wsb=need - 1) == wq.EWORKSPACE
    assert call(X=8) == wq.EALIGN
    assert call(layout=1, K=96) == wq.EUNSUPPORTED  # tiles need K % 128
    assert call(M=0) == wq.OK
