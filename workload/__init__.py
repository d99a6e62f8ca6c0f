"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This package holds only shapes and random numbers: no step of the attention
path is computed here.  Both the HIP path and the fp64 oracle consume exactly
what these generators return.
"""
from .configs import CONFIGS, Config, by_name, custom  # noqa: F401
from .gen import (  # noqa: F401
    TENSOR_IDS,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    gen_grad_outputs,
    gen_inputs,
    gen_tensor,
    outlier_rows,
    splitmix64,
)
