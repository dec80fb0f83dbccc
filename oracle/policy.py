"""Oracle of the draft-length policy: the next step's draft length K from the running acceptance
of past steps and the step costs.

TEST INFRASTRUCTURE ONLY: not imported by the HIP path.

The pages tie the best draft length to the hardware and the text: two drafted tokens on an
RTX 3050, one on a GTX 1650 Ti, and more gain on predictable text ("Gemma 4's MTP drafter
explained", sections "Tip: start with two drafted tokens" and "Why use a drafter?").  The reading
taken here: estimate the per-draft agreement probability p from past steps, then take the K that
maximises expected emitted tokens per unit time.

* A step that drafted K and accepted m drafts observed m agreements and, if m < K, one
  disagreement; drafts after it are never compared.  The likelihood p^m (1-p)^[m<K] gives the
  estimate p = (A + a0) / (A + R + a0 + r0), A = sum of m, R = number of steps with m < K, both
  decayed by a factor per step, a0 and r0 prior pseudo-counts.
* A step of K drafts emits 1 + p + ... + p^K tokens on average (the longest agreeing prefix plus
  the target's own token) and costs K drafter sub-steps plus a verify of K+1 rows, modelled as
  t_verify + K t_row.
"""

from __future__ import annotations

from dataclasses import dataclass


def expected_tokens(p: float, K: int) -> float:
    """1 + p + p^2 + ... + p^K, summed term by term."""
    total, term = 1.0, 1.0
    for _ in range(K):
        term *= p
        total += term
    return total


@dataclass
class KPolicy:
    k_min: int
    k_max: int
    decay: float
    prior_accepted: float
    prior_rejected: float
    t_draft_ms: float
    t_verify_ms: float
    t_row_ms: float
    accepted: float = 0.0
    rejected: float = 0.0

    def observe(self, K: int, n_emit) -> None:
        """One step that drafted K per sequence, with each sequence's emitted count."""
        acc = sum(n - 1 for n in n_emit)
        rej = sum(1 for n in n_emit if n - 1 < K)
        self.accepted = self.decay * self.accepted + acc
        self.rejected = self.decay * self.rejected + rej

    def acceptance(self) -> float:
        a = self.accepted + self.prior_accepted
        return a / (a + self.rejected + self.prior_rejected)

    def step_ms(self, K: int) -> float:
        return K * self.t_draft_ms + self.t_verify_ms + K * self.t_row_ms

    def choose(self) -> int:
        p = self.acceptance()
        rates = {K: expected_tokens(p, K) / self.step_ms(K) for K in range(self.k_min, self.k_max + 1)}
        best = max(rates.values())
        return min(K for K, r in rates.items() if r == best)
