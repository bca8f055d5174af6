"""CPU oracle for the speculative-decoding verifier.  TEST INFRASTRUCTURE ONLY.

A plain, slow fp64 NumPy statement of what the verifier computes, used to
check the HIP path.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does, and it shares no code with the HIP library.
"""

from .rejection_sampler import (  # noqa: F401
    RESIDUAL_Q_FLOOR,
    OracleOutputs,
    accept_ratio,
    acceptance_stats,
    draft_q_rows,
    decode_logits,
    greedy_tokens,
    inverse_cdf,
    residual_weights,
    target_distribution,
    verify,
)
