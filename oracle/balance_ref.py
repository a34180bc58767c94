"""Plain CPU oracle of the router balance step (float64 numpy).

Test infrastructure only, like the rest of ``oracle/``.

The pages warn that a routing balance score can improve while the actual
workload balance gets worse ("token gerrymandering", OC3 "Empirical findings
beyond raw speed"; TH "Scaling and optimising MoE training" says the same),
but they define neither the score nor a balance loss.  Plainest reading, and
the one taken here:

  f_e   = counts[e] / (T k)            share of the routed rows given to e
  P_e   = (1/T) sum_t p[t, e]          mean router probability of e
  score = E * sum_e f_e P_e            1 when both are uniform
  L_aux = alpha * score                the auxiliary load-balance loss

  actual balance = max_e counts[e] / mean_e counts[e]   (the busiest expert
                   sets the grouped GEMM's critical path; 1 when balanced)

Gradient: the indices (hence f) are not differentiable, so L_aux reaches the
router only through P:
  dL_aux / dp[t, e] = alpha * E * f_e / T  =: g_e        (same for every t)
and through the softmax like any other probability gradient:
  dlogits[t] = p[t] * (g - <p[t], g>).
The layer adds g_e to every token's gate-gradient row before the softmax
backward (``layer_backward(..., aux_alpha)`` in moe_ref).
"""

import numpy as np

F = np.float64


def balance(probs, counts, k, alpha, dtype=F):
    """Score, loss, the per-expert gradient coefficient g_e and the actual load
    balance of one routing step."""
    p = np.asarray(probs, dtype)
    c = np.asarray(counts, dtype)
    T, E = p.shape
    f = c / (T * k) if T > 0 else np.zeros(E, dtype)
    P = p.mean(axis=0) if T > 0 else np.zeros(E, dtype)
    score = E * float(np.sum(f * P))
    mean_load = T * k / E
    return dict(f=f, P=P, score=score, loss=alpha * score,
                g=(alpha * E * f / T) if T > 0 else np.zeros(E, dtype),
                max_over_mean=(float(c.max()) / mean_load) if T > 0 else 0.0)

