"""CPU oracle for fused scaled-dot-product attention (test infrastructure only).

This package is the slow, plain, obviously-correct fp64 definition that the HIP
kernels are checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product library never
imports, links or calls anything here, and nothing here imports the product
library: the two share no code. The only thing both sides consume is the seeded
input generator, which holds no attention arithmetic.

Modules
-------
``sdpa_reference``
    The definition: forward (output and per-row logsumexp) and the explicit
    backward formulas, in float64, one (batch, query-head) pair at a time.
``rounding_floor``
    A model of where a 16-bit matrix-core kernel must round (operands of the
    second and gradient products, stored outputs). It is used only to derive the
    unavoidable error floor that the parity tolerance is stated against; it is
    not an alternative definition of the result.

Parity status of each function is written in its module header.
"""

from .sdpa_reference import (  # noqa: F401
    attention_forward,
    attention_backward,
    head_forward,
    head_backward,
    group_backward,
)
from .rounding_floor import emulate_forward, emulate_backward, round_to  # noqa: F401
