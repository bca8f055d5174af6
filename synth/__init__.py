"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package holds input construction only: random target logits, draft
distributions, draft token ids and uniforms.  It contains none of the
verifier's own arithmetic (no acceptance test, no residual, no inverse-CDF
draw), so that the CPU oracle and the HIP path can both consume it without
sharing any of the method's code.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    WorkloadSpec,
    VerifyInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    make_config,
    make_point_config,
    make_sample_config,
    make_sparse_config,
    to_point,
    to_sparse,
)
