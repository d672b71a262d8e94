"""ctypes binding of libwq.so (C ABI in include/wq.h).

Argument marshalling only: every function with a ``wq_`` name forwards torch
tensors' device pointers and torch's current HIP stream to the C function of
the same name and turns a non-OK status into an exception.  All compute runs in
the HIP kernels of libwq.so; there is no fallback path.  The helpers below the
raw bindings (``quantize``, ``linear`` ...) only allocate outputs with torch
and chain the raw calls.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# WQ_LIB selects another build of the same C ABI (the CPU tests' sanitizer
# build of the host code); by default the in-tree gfx950 library is loaded.
LIB_PATH = os.environ.get("WQ_LIB") or os.path.join(HERE, "libwq.so")

FORMATS = {"bf16": 0, "int4": 1, "fp8": 2, "nvfp4": 3, "mxfp4": 4, "int4_asym": 5}
LAYOUT_ROWS, LAYOUT_TILES = 0, 1
OK, EINVAL, ESHAPE, EALIGN, EUNSUPPORTED, EWORKSPACE, EHIP = range(7)


class WQError(RuntimeError):
    """A non-OK status from libwq (``status`` holds the code)."""

    def __init__(self, status, name, detail):
        super().__init__("%s: %s" % (name, detail))
        self.status = status


class WQValueError(WQError, ValueError):
    pass


_lib = None


def lib():
    """Load libwq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libwq.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        L.wq_abi_version.restype = I
        L.wq_status_str.restype = ctypes.c_char_p
        L.wq_status_str.argtypes = [I]
        L.wq_last_error.restype = ctypes.c_char_p
        SP = ctypes.POINTER(ctypes.c_size_t)
        L.wq_layout.argtypes = [I, I64, I64, SP, SP, SP, SP]
        L.wq_quantize.argtypes = [I, P, I64, I64, P, P, P, P]
        L.wq_pack.argtypes = [I, P, I64, I64, P, P]
        I32 = ctypes.c_int32
        L.wq_dequantize.argtypes = [I, P, I32, P, P, I64, I64, P, P]
        L.wq_repack.argtypes = [I, I64, I64, I32, P, P, I32, P, P, P]
        L.wq_linear_workspace.argtypes = [I, I64, I64, I64]
        L.wq_linear_workspace.restype = SZ
        L.wq_linear.argtypes = [I, P, I64, I64, P, I32, P, P, P, I64, P, P, SZ, P]
        L.wq_linear_dq_gemm_workspace.argtypes = [I, I64, I64, I64]
        L.wq_linear_dq_gemm_workspace.restype = SZ
        L.wq_linear_dq_gemm.argtypes = [I, P, I64, I64, P, I32, P, P, P, I64, P, P, SZ, P]
        L.wq_absmax.argtypes = [P, I64, P, P]
        L.wq_fp8_scale.argtypes = [P, P, I64, P]
        L.wq_fp8_quantize_act.argtypes = [P, I64, I64, P, P, P]
        L.wq_fp8_static_workspace.argtypes = [I64, I64, I64]
        L.wq_fp8_static_workspace.restype = SZ
        L.wq_fp8_static_linear.argtypes = [P, I64, I64, P, P, I32, P, P, I64, P, P, SZ, P]
        L.wq_fp8_static_linear_noalloc.argtypes = [P, I64, I64, P, P, I32, P, P, I64, P, P]
        L.wq_fp8_linear_workspace.argtypes = [I64, I64, I64]
        L.wq_fp8_linear_workspace.restype = SZ
        L.wq_fp8_linear.argtypes = [P, I64, I64, P, P, I32, P, P, I64, P, P, SZ, P]
        L.wq_mx_quantize_act.argtypes = [P, I64, I64, P, P, P]
        L.wq_mx_linear.argtypes = [P, P, I64, I64, P, I32, P, P, I64, P, P]
        L.wq_mxfp4_dynamic_workspace.argtypes = [I64, I64]
        L.wq_mxfp4_dynamic_workspace.restype = SZ
        L.wq_mxfp4_dynamic_linear.argtypes = [P, I64, I64, P, I32, P, P, I64, P, P, SZ, P]
        L.wq_read_stream.argtypes = [P, SZ, P, P]
        L.wq_fp8_static_mlp2.argtypes = [P, I64, I64, P, P, P, P, I64, P, P, P, P, I64, P, P]
        L.wq_read_stream_words.argtypes = [SZ]
        L.wq_read_stream_words.restype = SZ
        for name in ("wq_layout", "wq_quantize", "wq_pack", "wq_repack", "wq_dequantize", "wq_linear",
                     "wq_linear_dq_gemm", "wq_absmax",
                     "wq_fp8_scale", "wq_fp8_quantize_act", "wq_fp8_static_linear", "wq_fp8_static_linear_noalloc",
                     "wq_fp8_linear",
                     "wq_read_stream", "wq_mx_quantize_act", "wq_mx_linear", "wq_mxfp4_dynamic_linear",
                     "wq_fp8_static_mlp2"):
            getattr(L, name).restype = I
        if L.wq_abi_version() != 2:
            raise RuntimeError("libwq ABI version mismatch")
        _lib = L
    return _lib


def _check(status, name):
    if status != OK:
        L = lib()
        detail = L.wq_last_error().decode()
        code = L.wq_status_str(status).decode()
        cls = WQError if status == EHIP else WQValueError
        raise cls(status, name, "%s (%s)" % (code, detail))


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# ---------------------------------------------------------------- raw bindings (same names as the C ABI)


def wq_abi_version():
    return lib().wq_abi_version()


def wq_layout(fmt, N, K):
    """-> (codes_bytes, packed_bytes, scale_bytes, global_bytes)"""
    out = [ctypes.c_size_t(0) for _ in range(4)]
    _check(lib().wq_layout(_fmt(fmt), N, K, *[ctypes.byref(o) for o in out]), "wq_layout")
    return tuple(o.value for o in out)


def wq_quantize(fmt, W, codes, scales, global_scale=None):
    N, K = W.shape
    _check(lib().wq_quantize(_fmt(fmt), _ptr(W), N, K, _ptr(codes), _ptr(scales), _ptr(global_scale),
                             _stream(W.device)), "wq_quantize")


def wq_pack(fmt, codes, packed):
    N, K = codes.shape
    _check(lib().wq_pack(_fmt(fmt), _ptr(codes), N, K, _ptr(packed), _stream(codes.device)), "wq_pack")


def wq_dequantize(fmt, packed, scales, global_scale, N, K, out, layout=LAYOUT_ROWS):
    _check(lib().wq_dequantize(_fmt(fmt), _ptr(packed), layout, _ptr(scales), _ptr(global_scale), N, K, _ptr(out),
                               _stream(out.device)), "wq_dequantize")


def wq_repack(fmt, N, K, src_layout, src_packed, src_scales, dst_layout, dst_packed, dst_scales):
    _check(lib().wq_repack(_fmt(fmt), N, K, src_layout, _ptr(src_packed), _ptr(src_scales), dst_layout,
                           _ptr(dst_packed), _ptr(dst_scales), _stream(src_packed.device)), "wq_repack")


def wq_linear_workspace(fmt, M, N, K):
    return lib().wq_linear_workspace(_fmt(fmt), M, N, K)


def wq_linear(fmt, X, packed, scales, global_scale, bias, N, Y, workspace=None, layout=LAYOUT_ROWS):
    M, K = X.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wq_linear(_fmt(fmt), _ptr(X), M, K, _ptr(packed), layout, _ptr(scales), _ptr(global_scale),
                           _ptr(bias), N, _ptr(Y), _ptr(workspace), ws_bytes, _stream(X.device)), "wq_linear")


def wq_linear_dq_gemm_workspace(fmt, M, N, K):
    return lib().wq_linear_dq_gemm_workspace(_fmt(fmt), M, N, K)


def wq_linear_dq_gemm(fmt, X, packed, scales, global_scale, bias, N, Y, workspace, layout=LAYOUT_ROWS):
    M, K = X.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wq_linear_dq_gemm(_fmt(fmt), _ptr(X), M, K, _ptr(packed), layout, _ptr(scales), _ptr(global_scale),
                                   _ptr(bias), N, _ptr(Y), _ptr(workspace), ws_bytes, _stream(X.device)),
           "wq_linear_dq_gemm")


def wq_absmax(X, amax):
    _check(lib().wq_absmax(_ptr(X), X.numel(), _ptr(amax), _stream(X.device)), "wq_absmax")


def wq_fp8_scale(amax, scale):
    _check(lib().wq_fp8_scale(_ptr(amax), _ptr(scale), amax.numel(), _stream(amax.device)), "wq_fp8_scale")


def wq_fp8_quantize_act(X, act_scale, Xq):
    M, K = X.shape
    _check(lib().wq_fp8_quantize_act(_ptr(X), M, K, _ptr(act_scale), _ptr(Xq), _stream(X.device)),
           "wq_fp8_quantize_act")


def wq_fp8_static_workspace(M, N, K):
    return lib().wq_fp8_static_workspace(M, N, K)


def wq_fp8_static_linear(X, act_scale, Wq, w_scale, bias, Y, workspace, layout=LAYOUT_ROWS):
    M, K = X.shape
    N = Wq.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wq_fp8_static_linear(_ptr(X), M, K, _ptr(act_scale), _ptr(Wq), layout, _ptr(w_scale), _ptr(bias),
                                      N, _ptr(Y), _ptr(workspace), ws_bytes, _stream(X.device)),
           "wq_fp8_static_linear")


def wq_fp8_static_linear_noalloc(X, act_scale, Wq, w_scale, bias, Y, layout=LAYOUT_ROWS):
    M, K = X.shape
    N = Wq.shape[0]
    _check(lib().wq_fp8_static_linear_noalloc(_ptr(X), M, K, _ptr(act_scale), _ptr(Wq), layout, _ptr(w_scale),
                                              _ptr(bias), N, _ptr(Y), _stream(X.device)),
           "wq_fp8_static_linear_noalloc")


def wq_fp8_linear_workspace(M, N, K):
    return lib().wq_fp8_linear_workspace(M, N, K)


def wq_fp8_linear(Xq, act_scale, Wq, w_scale, bias, Y, workspace=None, layout=LAYOUT_ROWS):
    M, K = Xq.shape
    N = Wq.shape[0]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wq_fp8_linear(_ptr(Xq), M, K, _ptr(act_scale), _ptr(Wq), layout, _ptr(w_scale), _ptr(bias), N,
                               _ptr(Y), _ptr(workspace), ws_bytes, _stream(Xq.device)), "wq_fp8_linear")


def wq_mx_quantize_act(X, Xq, Xs):
    M, K = X.shape
    _check(lib().wq_mx_quantize_act(_ptr(X), M, K, _ptr(Xq), _ptr(Xs), _stream(X.device)), "wq_mx_quantize_act")


def wq_mx_linear(Xq, Xs, K, Wq, Ws, bias, N, Y, layout=LAYOUT_ROWS):
    M = Xq.shape[0]
    _check(lib().wq_mx_linear(_ptr(Xq), _ptr(Xs), M, K, _ptr(Wq), layout, _ptr(Ws), _ptr(bias), N, _ptr(Y),
                              _stream(Xq.device)), "wq_mx_linear")


def wq_mxfp4_dynamic_workspace(M, K):
    return lib().wq_mxfp4_dynamic_workspace(M, K)


def wq_mxfp4_dynamic_linear(X, Wq, Ws, bias, N, Y, workspace, layout=LAYOUT_ROWS):
    M, K = X.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().wq_mxfp4_dynamic_linear(_ptr(X), M, K, _ptr(Wq), layout, _ptr(Ws), _ptr(bias), N, _ptr(Y),
                                         _ptr(workspace), ws_bytes, _stream(X.device)), "wq_mxfp4_dynamic_linear")


def wq_fp8_static_mlp2(X, act_scale1, W1q, w1_scale, b1, act_scale2, W2q, w2_scale, b2, Y):
    M, K1 = X.shape
    N1, N2 = W1q.shape[0], W2q.shape[0]
    _check(lib().wq_fp8_static_mlp2(_ptr(X), M, K1, _ptr(act_scale1), _ptr(W1q), _ptr(w1_scale), _ptr(b1), N1,
                                    _ptr(act_scale2), _ptr(W2q), _ptr(w2_scale), _ptr(b2), N2, _ptr(Y),
                                    _stream(X.device)), "wq_fp8_static_mlp2")


def wq_read_stream_words(nbytes):
    return lib().wq_read_stream_words(nbytes)


def wq_read_stream(buf, sink, nbytes=None):
    nbytes = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check(lib().wq_read_stream(_ptr(buf), nbytes, _ptr(sink), _stream(buf.device)), "wq_read_stream")


# ---------------------------------------------------------------- helpers: allocation + chaining

_WS = {}


def workspace(nbytes, device):
    """A uint8 workspace of at least `nbytes`, cached per (device, stream).
    It holds split-K partials and quantized activations, which need no
    initialisation, so it is reused."""
    if nbytes == 0:
        return None
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    t = _WS.get(key)
    if t is None or t.numel() < nbytes:
        # the caching allocator keeps a freed buffer for this stream until the
        # work queued on it has run, so growing needs no host synchronization
        t = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _WS[key] = t
    return t


def scale_dtype_shape(fmt, N, K):
    fmt = _fmt(fmt)
    if fmt == 1:
        return torch.bfloat16, (N, K // 128)
    if fmt == 2:
        return torch.float32, (N,)
    if fmt == 3:
        return torch.uint8, (N, K // 16)
    if fmt == 4:
        return torch.uint8, (N, K // 32)
    if fmt == 5:
        return torch.int32, (N, K // 128)  # uint32 words: bf16 scale | zero-point << 16
    return None, None


def quantize(fmt, W, layout=LAYOUT_ROWS):
    """Quantize bf16 W[N, K] on its device and pack it.  Returns a dict with
    codes (one per byte), packed, scales and global (NVFP4) tensors; with
    ``layout=LAYOUT_TILES`` the packed weight and scales are then converted to
    the kernel tile order (``wq_repack``) and the dict's ``layout`` says so."""
    f = _fmt(fmt)
    N, K = W.shape
    dev = W.device
    codes = torch.empty((N, K), dtype=torch.int8 if f == 1 else torch.uint8, device=dev)  # INT4_ASYM: 0..15
    sdt, sshape = scale_dtype_shape(f, N, K)
    scales = torch.empty(sshape, dtype=sdt, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev) if f == 3 else None
    wq_quantize(f, W, codes, scales, g)
    _, pb, _, _ = wq_layout(f, N, K)
    packed = torch.empty(pb, dtype=torch.uint8, device=dev).view(N, pb // N if N else 0)
    wq_pack(f, codes, packed)
    q = {"fmt": f, "N": N, "K": K, "codes": codes, "packed": packed, "scales": scales, "global": g,
         "layout": LAYOUT_ROWS}
    return repack(q, layout) if layout != LAYOUT_ROWS else q


def repack(q, layout):
    """A copy of quantize result `q` with its packed weight and scales in `layout`."""
    if q.get("layout", LAYOUT_ROWS) == layout:
        return q
    packed, scales = torch.empty_like(q["packed"]), torch.empty_like(q["scales"])
    wq_repack(q["fmt"], q["N"], q["K"], q.get("layout", LAYOUT_ROWS), q["packed"], q["scales"], layout, packed, scales)
    return dict(q, packed=packed, scales=scales, layout=layout)


def dequantize(q):
    out = torch.empty((q["N"], q["K"]), dtype=torch.bfloat16, device=q["packed"].device)
    wq_dequantize(q["fmt"], q["packed"], q["scales"], q["global"], q["N"], q["K"], out, q.get("layout", LAYOUT_ROWS))
    return out


def linear(X, q, bias=None, out=None):
    """Y = X . deq(W)^T (+ bias) with the fused dequant-GEMM.  `q` is a
    ``quantize`` result, or ``{"fmt": 0, "packed": W_bf16, "N": N, "K": K,
    "scales": None, "global": None}`` for the dense bf16 Linear."""
    M, K = X.shape
    N = q["N"]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    ws = workspace(wq_linear_workspace(q["fmt"], M, N, K), X.device)
    wq_linear(q["fmt"], X, q["packed"], q["scales"], q["global"], bias, N, out, ws, q.get("layout", LAYOUT_ROWS))
    return out


def linear_two_kernel(X, q, bias=None, out=None):
    """The two-kernel form (``wq_linear_dq_gemm``): dequantize to bf16, then the
    dense bf16 GEMM."""
    M, K = X.shape
    N = q["N"]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    ws = workspace(wq_linear_dq_gemm_workspace(q["fmt"], M, N, K), X.device)
    wq_linear_dq_gemm(q["fmt"], X, q["packed"], q["scales"], q["global"], bias, N, out, ws,
                      q.get("layout", LAYOUT_ROWS))
    return out


def dense(W):
    """Wrap a bf16 weight as the unquantized format (for ``linear``)."""
    N, K = W.shape
    return {"fmt": 0, "N": N, "K": K, "codes": None, "packed": W, "scales": None, "global": None,
            "layout": LAYOUT_ROWS}


def static_fp8_linear(X, act_scale, Wq, w_scale, bias=None, out=None, layout=LAYOUT_ROWS):
    M, K = X.shape
    N = Wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    ws = workspace(wq_fp8_static_workspace(M, N, K), X.device)
    wq_fp8_static_linear(X, act_scale, Wq, w_scale, bias, out, ws, layout)
    return out


def mx_quantize_act(X):
    """Dynamic MX quantization of bf16 X [M, K] -> (packed codes [M, K/2], E8M0 scales [M, K/32])."""
    M, K = X.shape
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    Xs = torch.empty((M, K // 32), dtype=torch.uint8, device=X.device)
    wq_mx_quantize_act(X, Xq, Xs)
    return Xq, Xs


def mxfp4_dynamic_linear(X, q, bias=None, out=None):
    """Y = MX(X) . deq(W)^T (+ bias) on the scaled fp4 matrix cores; `q` is a
    ``quantize("mxfp4", W)`` result."""
    M, K = X.shape
    N = q["N"]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    ws = workspace(wq_mxfp4_dynamic_workspace(M, K), X.device)
    wq_mxfp4_dynamic_linear(X, q["packed"], q["scales"], bias, N, out, ws, q.get("layout", LAYOUT_ROWS))
    return out


def calibrate_act_scale(batches_or_inputs):
    """Absmax observer over a list of bf16 device tensors -> act_scale (device
    float tensor of 1) = amax / 448."""
    dev = batches_or_inputs[0].device
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    for x in batches_or_inputs:
        wq_absmax(x, amax)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    wq_fp8_scale(amax, scale)
    return scale, amax
