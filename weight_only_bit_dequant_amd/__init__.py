"""MI355X (gfx950) weight-only low-bit quantized Linear and static-FP8 Linear.

The compute lives in the HIP library ``libwq.so`` (C ABI declared in
``include/wq.h``); ``weight_only_bit_dequant_amd.wq`` is the thin ctypes
binding.  Importing this package loads nothing; the first call into ``wq``
loads the library and raises if it is missing.
"""

__all__ = ["synth", "wq"]
