"""The nn.Module front end (weight_only_bit_dequant_amd/modules.py) on the
pages' toy models: the swapped modules call the same kernels as the raw entry
points (bit-identical outputs) and match the oracle within the bar."""

import numpy as np
import pytest
import torch

from oracle import gemm as G
from oracle import mx_dynamic as MX
from oracle import quant as Q
from oracle import static_fp8 as S
from oracle import codecs as C
from weight_only_bit_dequant_amd import synth

wq = pytest.importorskip("weight_only_bit_dequant_amd.wq")
modules = pytest.importorskip("weight_only_bit_dequant_amd.modules")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


class Toy(torch.nn.Module):
    """The weight-only pages' model: one nn.Linear(3072, 4096) with bias."""

    def __init__(self, W, b):
        super().__init__()
        self.linear = torch.nn.Linear(W.shape[1], W.shape[0], bias=b is not None, dtype=torch.bfloat16, device=DEV)
        with torch.no_grad():
            self.linear.weight.copy_(synth.as_torch_bf16(W, DEV))
            if b is not None:
                self.linear.bias.copy_(synth.as_torch_bf16(b, DEV))

    def forward(self, x):
        return self.linear(x)


def rel(Y, ref):
    return G.rel_frobenius(C.bf16_to_f32(synth.from_torch_bf16(Y.reshape(-1, Y.shape[-1]))).astype(np.float64), ref)


@pytest.mark.parametrize("fmt,fn", [("int4", "quantize_linear_int4_symmetric"), ("nvfp4", "quantize_linear_nvfp4"),
                                    ("fp8", "quantize_linear_fp8_weight_only"), ("mxfp4", "quantize_linear_mxfp4")])
def test_weight_only_swap(fmt, fn):
    W, b, X = synth.linear_case(512, 768, 32, cfg=60)
    model = Toy(W, b)
    getattr(modules, fn)(model)
    assert isinstance(model.linear, modules.QuantizedLinear)
    x = synth.as_torch_bf16(X, DEV).reshape(4, 8, 768)  # leading dims are flattened and restored
    y = model(x)
    assert y.shape == (4, 8, 512)
    raw = wq.linear(synth.as_torch_bf16(X, DEV), model.linear.q, synth.as_torch_bf16(b, DEV))
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(32, 512).view(torch.int16), raw.view(torch.int16))
    codes, scales, g = Q.quantize(fmt, W)
    assert rel(y, G.linear_fp64(X, Q.dequant(fmt, codes, scales, g), b)) <= 1e-2


def test_mxfp4_dynamic_swap():
    W, b, X = synth.linear_case(512, 768, 32, cfg=61)
    model = Toy(W, b)
    modules.quantize_linear_mxfp4(model, dynamic_activation=True)
    y = model(synth.as_torch_bf16(X, DEV))
    torch.cuda.synchronize()
    wc, ws = Q.quantize_mxfp4(W)
    assert rel(y, MX.forward(X, wc, ws, b)) <= 1e-2


def test_static_fp8_swap_two_layer():
    """The static page's MLP, calibrated on its 10 seeded batches."""
    weights = synth.mlp_weights()
    batches = synth.calibration_batches(32, 256)
    model = torch.nn.Sequential(torch.nn.Linear(256, 512, bias=False), torch.nn.Linear(512, 128, bias=False))
    model = model.to(device=DEV, dtype=torch.bfloat16)
    with torch.no_grad():
        for lin, w in zip(model, weights):
            lin.weight.copy_(synth.as_torch_bf16(w, DEV))
    # calibration runs the float model (torch's bf16 nn.Linear); the scales
    # it yields are then used on both sides
    modules.quantize_static_fp8(model, None, calibration_batches=[(synth.as_torch_bf16(bb, DEV),) for bb in batches])
    assert all(isinstance(m, modules.StaticFP8Linear) for m in model)
    x = synth.activations(32, 256, synth.SEED_X + 5)
    y = model(synth.as_torch_bf16(x, DEV))
    torch.cuda.synchronize()
    s1 = np.float32(model[0].act_scale.cpu().numpy()[0])
    s2 = np.float32(model[1].act_scale.cpu().numpy()[0])
    # layer-1 scale: exact (observed on the inputs themselves)
    assert s1 == S.scale_from_amax(max(S.absmax(bb) for bb in batches))
    qref = S.quantize_model(weights)
    y_ref, _ = S.quant_forward(x, [s1, s2], qref)
    assert rel(y, y_ref) <= 1e-2


def test_modules_refuse_cpu_and_fp32():
    W, b, X = synth.linear_case(64, 128, 4, cfg=62)
    model = Toy(W, b)
    modules.quantize_linear_int4_symmetric(model)
    with pytest.raises(TypeError):
        model(torch.zeros(4, 128, dtype=torch.float32, device=DEV))
    with pytest.raises(RuntimeError):
        model.linear(torch.zeros(4, 128, dtype=torch.bfloat16))
