"""CPU oracle for paged fp8-KV attention (decode and causal prefill).

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, float64 definition
that the HIP library is checked against.  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import it;
the library and its binding never do, and the two share no code.

Modules:
  fp8        exact 256-code decode tables of OCP e4m3 and e5m2, built two ways.
  attention  the attention definition over a paged cache, and the state merge.

Every function here is pinned by tests under ``tests/`` (test_oracle_*.py) to
something other than itself: the two table constructions against each other and
against fixed anchor codes; the attention against brute-force scalar loops on
tiny inputs, closed forms and invariants.  No function is "parity unpinned".
"""
from . import attention, fp8  # noqa: F401
