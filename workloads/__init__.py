"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This package only draws random bf16 tensors of the shapes and distributions of
the diffusion-transformer linears the pages measure; it holds none of the
method's arithmetic (no quantisation, no product, no epilogue). Both the HIP
path and the CPU oracle receive the very same bf16 bytes from here.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    LinearCase,
    bf16_bits,
    make_case,
    make_config,
    layer_specs,
)
