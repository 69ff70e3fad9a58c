"""fp64 CPU oracle for exact backward-over-backward through softmax attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library. It shares no code with the
HIP path. Every function in it is pinned by the CPU tests (finite differences,
closed forms, invariants, an independent symbolic derivation and an independent
autograd implementation); no function here is "parity unpinned".
"""

from .bob import (  # noqa: F401
    attention_forward,
    attention_forward_head,
    bob,
    bob_cols_head,
    bob_head,
    bob_rows_head,
    first_backward,
    first_backward_head,
)
