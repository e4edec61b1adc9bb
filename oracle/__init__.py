"""CPU oracle for the FP8 W8A8 linear layer (test infrastructure, not product code).

This package is the plain, slow, obviously correct statement of what the GPU path
computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it, call it or load anything built from it. The HIP
library under ``fp8_w8a8_quantized_token_amd`` never imports it, and this package
imports nothing from there: the two share no code, headers, tables or helpers.

Method (HunyuanVideo1.5 BF16->FP8 retrospective, aigcage.com/blog/hunyuanvideo-fp8,
section 3.1): a bf16 activation is quantised per token (row) at run time to FP8
E4M3, multiplied by an FP8 weight that was quantised per output channel ahead of
time (section 2 of the same page), and the product is scaled, biased and written
in the output dtype.

Modules
  e4m3    decode / round-to-nearest-even saturating encode of OCP e4m3fn codes
  quant   per-row (per-token, per-channel) amax -> scale -> code quantisation
  linear  exact float64 FP8 product and the scale/bias epilogue
  act     GELU / SiLU rounded exactly to bf16 (the producer upstream of the FFN-down
          linear), then the per-token quantiser: the fused producer's result
  e5m2    decode / round-to-nearest-even saturating encode of OCP e5m2 codes
  tensor_quant  per-tensor quantisation (either format) and fp32 dequantisation
  w8a16   the FP8 weight-only linear: bf16 activation times the per-channel e4m3fn
          weight, in float64

Every function here is pinned by tests under ``tests/`` against facts fixed
outside this package (the format definition, torch's CPU float8 cast, brute
force, closed forms and invariants); nothing here is "parity unpinned".
"""

from . import e4m3, e5m2, quant, linear, act, w8a16, tensor_quant  # noqa: F401

__all__ = ["e4m3", "e5m2", "quant", "linear", "act", "w8a16", "tensor_quant"]
