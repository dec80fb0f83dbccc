"""CPU oracle for greedy speculative decoding with an MTP drafter.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 numpy code written from the
pages' description of the method, used to check the HIP path.  Only the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the HIP library or its
Python binding; both sides take their seeded inputs from ``workloads``.

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (closed forms, textbook special cases, brute force, the
invariants the pages state, an independent matrix-form forward).  The drafter
layer numerics (``draft``) are pinned only by special cases and by
self-consistency; there is no printed worked example on the pages.
"""

from .model import *  # noqa: F401,F403
