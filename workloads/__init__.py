"""Seeded synthetic inputs for the LiftQuant decode operator.

This package only draws random numbers and converts them to the storage
dtypes the operator consumes. It holds none of the operator's arithmetic, so
both the CPU oracle (``oracle/``) and the HIP path (``bit_matmul_amd``) may
use it without sharing any of the method's code.
"""
from .configs import LayerSpec, Workload, WORKLOADS, workload, all_layers
from .gen import (
    LayerInputs,
    make_layer,
    make_layer_small,
    bf16_round,
    bf16_bits,
    sign_bits_to_int8,
)

__all__ = [
    "LayerSpec", "Workload", "WORKLOADS", "workload", "all_layers",
    "LayerInputs", "make_layer", "make_layer_small",
    "bf16_round", "bf16_bits", "sign_bits_to_int8",
]
