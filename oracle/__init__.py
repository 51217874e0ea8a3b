"""fp64 CPU oracle for the fused SwiGLU MLP (test infrastructure only).

This package is the reference that the HIP path is checked against. It is
test infrastructure: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product package
(``backward_gate_up_amd``) never imports it, and this package imports
nothing from the product package; the two share no code.

Everything here is plain numpy float64 (plus ``@`` for the matrix products),
applied to the exact values of the low-precision inputs, with no
intermediate rounding unless a function says it rounds.

Sources (the pages):
  * "[RFC] Full-pipeline SwiGLU MLP with forward/backward co-optimization"
    (Liger-Kernel issue #1347), section "Summary": the dataflow and the names
    A, G, U, dA, dG, dU and dI; section "Correctness": the output set Y, dI,
    dWg, dWu, dWd.
  * "Scope one-round FP32 SwiGLU to the exact Qwen3.5 contract" (xorl PR #51),
    review thread: the one-round program (SiLU and the product in fp32,
    rounded once to the output dtype) versus the historical two-round one.

The pages never write out SiLU or its derivative; the textbook forms are used.

Parity status per function is listed in ``oracle.swiglu.PARITY``.
"""

from .swiglu import (  # noqa: F401
    PARITY,
    sigmoid,
    silu,
    silu_prime,
    fwd,
    bwd,
    infer,
    fwd_naive,
    bwd_naive,
    rows,
    cols,
    epilogue_fwd,
    epilogue_fwd_two_round,
    epilogue_bwd,
)
from .rounding import round_to, ulp_distance, ordered_int  # noqa: F401
