"""Seeded synthetic workloads shared by the oracle side and the GPU side.

This package generates *inputs* only: weights, KV caches, hidden states,
prompts and the counter-based random numbers that the speculative loop's
draft injection draws.  It holds none of the decoding method's arithmetic
(no norms, attention, projections, argmax or acceptance).  Both the CPU
oracle (``oracle/``) and the HIP path's tests and benchmark import it; the
device-side fill library under ``workloads/csrc`` implements the same
counter-based generator from the same published definition, so large
configurations can be generated on the GPU bit-identically.
"""

from .synth import *  # noqa: F401,F403
from .configs import *  # noqa: F401,F403
