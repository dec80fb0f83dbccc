"""CPU oracle for greedy speculative decoding with an MTP drafter.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy code written from the
pages' description of the method, used to check the HIP path.  Only the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the HIP library or its
Python binding; both sides take their seeded inputs from ``workloads``.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (closed forms, textbook special cases, brute force, the
invariants the pages state, an independent matrix-form forward).  The drafter
sub-step (``drafter_substep`` / ``draft``) is pinned by hand-worked closed
forms on 2-wide weights and by an independent explicit-loop drafter, and each
plausible wiring mistake planted into a copy of this source fails one of those
pins (tests/test_oracle_drafter.py); the pages print no worked example.
"""

from .model import *  # noqa: F401,F403
from .policy import KPolicy, expected_tokens  # noqa: F401
