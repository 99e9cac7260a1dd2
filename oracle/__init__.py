"""Plain fp64 CPU oracle for sparse top-k MLA attention (DeepSeek sparse attention).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, calls or links anything here.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

Modules
-------
``smla``   per-token, per-slot definition of the forward and backward
           (``oracle_fwd``, ``oracle_bwd``) and of the exact Delta
           (``oracle_delta_exact``) and of the sink gradient alone (``oracle_dsink``),
           written out in fp64 NumPy.
``dense``  a second, independent formulation: dense masked attention over all
           KV rows in torch fp64, with autograd gradients.  It pins ``smla``.
``fd``     central finite differences of L = sum(dO * O), a third pin that
           needs neither formulation's gradient code.

Parity status: every function here is pinned by tests under ``tests/``
(dense brute force, finite differences, closed forms and invariants); the one
thing left unpinned is the exact fp32 summation order and the bf16 bit patterns
of the GPU outputs, which no definition fixes (compared to tolerance only).
"""
from .smla import (  # noqa: F401
    valid_slots,
    glae,
    p_sink,
    round_to_bf16,
    oracle_fwd,
    oracle_bwd,
    oracle_delta_exact,
    oracle_dsink,
)
