"""nn.Module front end: in-place module swaps with the pages' call shapes.

Each page quantizes a model in place and then calls it:
  * INT4 page, "Quantize weights to symmetric INT4":
    ``quantize_linear_int4_symmetric(model, group_size=128)``
  * NVFP4 page, "Quantize weights to NVFP4": ``quantize_linear_nvfp4(model)``
  * FP8 page, "Quantize weights to FP8": ``quantize_(model, Float8WeightOnlyConfig())``
    -> here ``quantize_linear_fp8_weight_only(model)``
  * MXFP4 page, "Quantize weights to MXFP4": ``quantize_linear_mxfp4(model)``
    (``dynamic_activation=True`` also quantizes activations to MX per call,
    the page title's "Dynamic Activation + MX Weight" config)
  * Static FP8 page, "Calibrate, then insert static FP8 Q/DQ":
    ``quantize_static_fp8(model, (example_input,), calibration_steps=10)``

Every ``nn.Linear`` in the model is replaced by a module that holds the packed
weight and runs the library's kernels in ``forward``; the weight is packed once
and never refit.  Modules run on the GPU only: there is no CPU path.
"""

import torch

from . import wq

_CODES = {"int4": "int4", "nvfp4": "nvfp4", "fp8": "fp8", "mxfp4": "mxfp4"}


def _as_2d(x):
    if x.dtype != torch.bfloat16:
        raise TypeError("quantized linear layers take bf16 activations (got %s)" % x.dtype)
    if not x.is_cuda:
        raise RuntimeError("quantized linear layers run on the GPU only")
    lead = x.shape[:-1]
    return x.reshape(-1, x.shape[-1]).contiguous(), lead


def _bias(linear):
    return None if linear.bias is None else linear.bias.detach().to(torch.bfloat16).contiguous()


class QuantizedLinear(torch.nn.Module):
    """Weight-only low-bit Linear: y = x . deq(W)^T + b with the dequantization
    fused ahead of the bf16 matrix multiply (``wq_linear``)."""

    def __init__(self, linear, fmt):
        super().__init__()
        if fmt not in _CODES:
            raise ValueError("unknown format %r" % (fmt,))
        w = linear.weight.detach().to(torch.bfloat16).contiguous()
        self.fmt = fmt
        self.in_features, self.out_features = linear.in_features, linear.out_features
        self.q = wq.quantize(fmt, w)
        self.bias = _bias(linear)

    def forward(self, x):
        x2, lead = _as_2d(x)
        y = wq.linear(x2, self.q, self.bias)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self):
        return "in_features=%d, out_features=%d, format=%s" % (self.in_features, self.out_features, self.fmt)


class MXDynamicLinear(QuantizedLinear):
    """MXFP4 weight x activations quantized to MX on every call, multiplied on
    the scaled fp4 matrix cores (``wq_mxfp4_dynamic_linear``)."""

    def __init__(self, linear):
        super().__init__(linear, "mxfp4")

    def forward(self, x):
        x2, lead = _as_2d(x)
        y = wq.mxfp4_dynamic_linear(x2, self.q, self.bias)
        return y.reshape(*lead, self.out_features)


class StaticFP8Linear(torch.nn.Module):
    """Static FP8 Linear: activation Q with a calibrated per-tensor scale, then
    the E4M3 x E4M3 GEMM (``wq_fp8_static_linear``)."""

    def __init__(self, linear, act_scale):
        super().__init__()
        w = linear.weight.detach().to(torch.bfloat16).contiguous()
        self.in_features, self.out_features = linear.in_features, linear.out_features
        self.q = wq.quantize("fp8", w)
        self.act_scale = act_scale
        self.bias = _bias(linear)

    def forward(self, x):
        x2, lead = _as_2d(x)
        y = wq.static_fp8_linear(x2, self.act_scale, self.q["codes"], self.q["scales"], self.bias)
        return y.reshape(*lead, self.out_features)


def _swap(model, make):
    """Replace every nn.Linear under `model` (in place) by make(linear, name)."""
    if isinstance(model, torch.nn.Linear):
        raise TypeError("pass a container module; a bare nn.Linear cannot be swapped in place")
    for name, child in list(model.named_children()):
        if isinstance(child, torch.nn.Linear):
            setattr(model, name, make(child, name))
        else:
            _swap(child, make)
    return model


def quantize_linear_int4_symmetric(model, group_size=128):
    if group_size != 128:
        raise ValueError("the INT4 kernels use group_size=128")
    return _swap(model, lambda lin, _: QuantizedLinear(lin, "int4"))


def quantize_linear_nvfp4(model):
    return _swap(model, lambda lin, _: QuantizedLinear(lin, "nvfp4"))


def quantize_linear_fp8_weight_only(model):
    return _swap(model, lambda lin, _: QuantizedLinear(lin, "fp8"))


def quantize_linear_mxfp4(model, dynamic_activation=False):
    if dynamic_activation:
        return _swap(model, lambda lin, _: MXDynamicLinear(lin))
    return _swap(model, lambda lin, _: QuantizedLinear(lin, "mxfp4"))


@torch.no_grad()
def quantize_static_fp8(model, example_inputs, calibration_steps=10, calibration_batches=None):
    """Calibrate per-tensor activation scales with absmax observers on the
    float model (``calibration_steps`` forwards), then swap every nn.Linear for
    a StaticFP8Linear.  `calibration_batches` (a list of input tuples) replaces
    the repeated example input when given."""
    amax = {}
    hooks = []
    for name, mod in model.named_modules():
        if isinstance(mod, torch.nn.Linear):

            def hook(m, inputs, name=name):
                x = inputs[0]
                if x.dtype != torch.bfloat16 or not x.is_cuda:
                    raise TypeError("calibration inputs must be bf16 GPU tensors")
                a = amax.get(name)
                if a is None:
                    a = torch.zeros(1, dtype=torch.float32, device=x.device)
                    amax[name] = a
                wq.wq_absmax(x.contiguous(), a)

            hooks.append(mod.register_forward_pre_hook(hook))
    try:
        batches = calibration_batches if calibration_batches is not None else [example_inputs] * calibration_steps
        for inp in batches:
            model(*inp)
    finally:
        for h in hooks:
            h.remove()
    scales = {}
    for name, a in amax.items():
        s = torch.empty(1, dtype=torch.float32, device=a.device)
        wq.wq_fp8_scale(a, s)
        scales[name] = s

    # swap, keyed by the full module path the observers used
    def swap(mod, prefix):
        for cname, child in list(mod.named_children()):
            full = prefix + cname
            if isinstance(child, torch.nn.Linear):
                if full not in scales:
                    raise RuntimeError("layer %s saw no calibration input" % full)
                setattr(mod, cname, StaticFP8Linear(child, scales[full]))
            else:
                swap(child, full + ".")

    swap(model, "")
    return model
