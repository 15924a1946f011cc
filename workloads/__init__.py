"""Seeded synthetic inputs for the sparse MoE layer forward.

This package only draws numbers: activations, router and expert weights, router
biases, the low-bit encodings of expert weights and the sparsity thresholds
(layer parameters calibrated offline on a seeded batch).  It contains none of
the layer's arithmetic (no logits, no top-k, no permutation, no FFN, no
dequantisation), so both the CPU oracle and the HIP path may import it.
"""
from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401
from .gen import Workload, make_workload, bf16_bits_to_f32, f32_to_bf16_bits  # noqa: F401
from .gen import Replica, make_replica, MwqWeights, quantize_mwq_rows  # noqa: F401
from .gen import Int2Weights, quantize_int2_rows, sparsity_thresholds  # noqa: F401
