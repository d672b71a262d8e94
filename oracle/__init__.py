"""CPU oracle for the weight-only low-bit quantized Linear and the static-FP8 Linear.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``weight_only_bit_dequant_amd``) and never imports it.

What it implements, and from which passage (the pages are the Torch-TensorRT
"TorchAO ... (Linear)" tutorials; each function names its page and section):

* ``codecs``  -- bf16 <-> fp32, E4M3 (OCP "fn"), E2M1, E8M0 and INT4 decode and
  round-to-nearest-even saturating encoders.  The pages only name these formats
  (NVFP4 page, intro: packed E2M1 + E4M3 block scales + FP32 global scale;
  MXFP4 page, intro: E2M1 + E8M0 block scales, block 32; static FP8 page,
  intro: e4m3).  The value sets follow the OCP OFP8 and OCP MX v1.0 format
  definitions.
* ``quant``   -- the four weight quantizers, nibble packing and dequantization.
* ``gemm``    -- the fp64 Linear (Y = X deq(W)^T + b), relative Frobenius
  error and the page's ``sqnr`` helper.
* ``static_fp8`` -- calibration (absmax observers), activation Q and the
  static-FP8 Linear / two-layer model.
* ``mx_dynamic`` -- dynamic MX quantization of activations and the MXFP4 x
  MXFP4 Linear of the MXFP4 page's "Dynamic Activation + MX Weight" config.

Arithmetic rules used throughout: bf16 inputs widen exactly to fp32; every
quantizer step is an IEEE fp32 operation (numpy float32, correctly rounded);
every cast to a low-bit code clamps to the format's largest finite magnitude and
then rounds to nearest, ties to even, keeping the sign (so -0 and -tiny give a
negative-zero code); dequantized values and the GEMM are evaluated in fp64,
where every dequantized weight is exact.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library casts, brute force or invariants, except the
static-FP8 end-to-end SQNR *value*, which the pages do not print
("parity unpinned": only its own consistency is checked).
"""

from . import codecs, quant, gemm, static_fp8  # noqa: F401
