"""Seeded synthetic inputs for the paged-KV decode path.

This package only draws numbers: sequence lengths, the pool's allocation
order, K/V histories and queries. It holds none of the method's arithmetic
(no allocation, no indexing, no attention), so both the CPU oracle and the
HIP library can consume the same inputs without sharing any computation.
"""
from .synth import (  # noqa: F401
    BF16,
    F32,
    Workload,
    build_workload,
    config_workload,
    CONFIG_NAMES,
    f32_to_bf16_bits,
    poison_bits,
)
from .forks import ForkWorkload, best_of_n_workload, build_fork_workload  # noqa: F401
from .speculative import SpecWorkload, build_spec_workload, verify_workload  # noqa: F401
from .sampling import SampleWorkload, build_sample_workload, lm_head_workload  # noqa: F401
