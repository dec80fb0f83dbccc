// Draft-length policy (host code): the next step's K from the running acceptance of past steps
// and the measured cost of drafting and verifying.
//
// A step that drafts K tokens and accepts m of them has seen m drafts agree and, when m < K, one
// disagree; the drafts after the first disagreement say nothing.  Under a per-draft agreement
// probability p the step's likelihood is p^m (1 - p)^[m < K], so over many steps the maximum-
// likelihood p is (sum of m) / (sum of m + number of steps with m < K).  The counts decay by a
// fixed factor per step so that the estimate follows the text (the pages note that the gain
// depends on what is being written), and pseudo-counts keep it away from 0 and 1 at the start.
//
// With p, a step of K drafts emits 1 + p + ... + p^K tokens on average and costs K drafter
// sub-steps plus a verify of K + 1 rows, modelled as t_verify + K t_row.  The policy takes the K
// in [k_min, k_max] with the most tokens per unit time (the smallest such K on a tie).

#include "../../include/specdec.h"

#include <cmath>

namespace {

bool finite_pos(float v) { return std::isfinite(v) && v >= 0.f; }

// Expected tokens per step and time per step of a draft length K.
double step_tokens(double p, int K) {
  double e = 1.0, pj = 1.0;
  for (int j = 1; j <= K; ++j) {
    pj *= p;
    e += pj;
  }
  return e;
}

}  // namespace

extern "C" {

int specdec_k_policy_init(specdec_k_policy* pol, int32_t k_min, int32_t k_max, float decay,
                          float prior_accepted, float prior_rejected, float t_draft_ms,
                          float t_verify_ms, float t_row_ms) {
  if (!pol || k_min < 1 || k_max < k_min) return SPECDEC_E_INVAL;
  if (!(decay > 0.f && decay <= 1.f)) return SPECDEC_E_INVAL;
  if (!(prior_accepted > 0.f) || !(prior_rejected > 0.f) || !std::isfinite(prior_accepted) ||
      !std::isfinite(prior_rejected))
    return SPECDEC_E_INVAL;
  if (!finite_pos(t_draft_ms) || !(t_verify_ms > 0.f) || !std::isfinite(t_verify_ms) ||
      !finite_pos(t_row_ms))
    return SPECDEC_E_INVAL;
  pol->k_min = k_min;
  pol->k_max = k_max;
  pol->decay = decay;
  pol->prior_accepted = prior_accepted;
  pol->prior_rejected = prior_rejected;
  pol->t_draft_ms = t_draft_ms;
  pol->t_verify_ms = t_verify_ms;
  pol->t_row_ms = t_row_ms;
  pol->accepted = 0.0;
  pol->rejected = 0.0;
  return SPECDEC_OK;
}

int specdec_k_policy_observe(specdec_k_policy* pol, int32_t K, const int32_t* n_emit, int32_t B) {
  if (!pol || !n_emit || B < 1 || K < 1) return SPECDEC_E_INVAL;
  for (int b = 0; b < B; ++b)
    if (n_emit[b] < 1 || n_emit[b] > K + 1) return SPECDEC_E_INVAL;
  double acc = 0.0, rej = 0.0;
  for (int b = 0; b < B; ++b) {
    const int m = n_emit[b] - 1;  // drafts accepted
    acc += m;
    rej += m < K ? 1.0 : 0.0;
  }
  pol->accepted = pol->decay * pol->accepted + acc;
  pol->rejected = pol->decay * pol->rejected + rej;
  return SPECDEC_OK;
}

double specdec_k_policy_acceptance(const specdec_k_policy* pol) {
  if (!pol) return -1.0;
  const double a = pol->accepted + pol->prior_accepted;
  return a / (a + pol->rejected + pol->prior_rejected);
}

int32_t specdec_k_policy_choose(const specdec_k_policy* pol) {
  if (!pol) return SPECDEC_E_INVAL;
  const double p = specdec_k_policy_acceptance(pol);
  int best = pol->k_min;
  double best_rate = -1.0;
  for (int K = pol->k_min; K <= pol->k_max; ++K) {
    const double t = (double)K * pol->t_draft_ms + pol->t_verify_ms + (double)K * pol->t_row_ms;
    const double rate = step_tokens(p, K) / t;
    if (rate > best_rate) {
      best_rate = rate;
      best = K;
    }
  }
  return best;
}

}  // extern "C"
