"""Float64 CPU oracle for the GatedDeltaNet operator.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The operator library
never calls it, and it shares no code with the HIP path.

Parity: every function here is pinned by the CPU test suite against closed
forms, invariants and brute-force reformulations (see tests/test_oracle_pins.py).
"""
from .gdn_oracle import (  # noqa: F401
    softplus, log_decay, gates, l2normalize, key_head_index, capsule_width,
    capsule_sections, recurrence, gdn_forward, gdn_replay, chunk_step,
    chunked_forward, L2NORM_EPS,
)
