"""Seeded synthetic inputs shared by the oracle tests and the HIP path.

This package draws random numbers and shapes them into the five benchmark
workloads (tensor shapes, value distributions, planted outlier dimensions,
group layouts and raw coefficient draws).  It performs none of the attention
method's own arithmetic: no scores, kernels, feature maps, states, contribution
statistics or coefficient mappings live here.
"""

from .workloads import (  # noqa: F401
    CONFIG_NAMES,
    Workload,
    bf16_round,
    make,
    decode_prefix_lengths,
    calibration_plan,
)
