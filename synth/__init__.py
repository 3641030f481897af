"""Seeded synthetic inputs for exact attention.

This package only draws random numbers and shapes them into the workloads the
tests and the benchmark run. It holds none of the attention arithmetic: no
scores, softmax, masks applied to scores or gradients. Both the CPU oracle side
(tests) and the GPU side (tests, bench) take their inputs from here.
"""

from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    normal,
    qkv_inputs,
    key_ranges,
    seed_for,
    with_outliers,
    random_signs,
    bias_tensor,
)
