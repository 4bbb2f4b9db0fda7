"""Error budgets shared by the GPU parity tests (test infrastructure: oracle
quantities only, no GPU result enters a bound)."""

import numpy as np

from oracle import naive_probs

BF16_U = 2.0 ** -8   # bf16 unit roundoff: 8 significant bits


def d_term_bounds(q, k, v, do, scale, causal):
    """Per-element bounds (first order, from oracle quantities of one head) on
    what the forward's bf16 output adds to the backward's dQ and dK errors.

    The backward forms D_i = sum_c dO_ic O_ic from the O the forward stored
    ("FlashAttention from scratch", Step 4: D from the saved output), which
    differs from the exact O by its own rounding (<= u |O|) and by the rounding
    of each probability to bf16 before the P V product (<= u P|V|):
    |D^_i - D_i| <= sum_c |dO_ic| u (|O_ic| + (P|V|)_ic) = delta_i.  With
    dS = P (dP - D), dK_j = scale sum_i dS_ij Q_i and dQ_i = scale sum_j dS_ij K_j
    move by at most |scale| sum_i P_ij delta_i |Q_i| and
    |scale| delta_i sum_j P_ij |K_j|.  q, k, v, do: [N, d] of one head.
    Returns (bound on dQ, bound on dK), each [N, d].
    """
    P = naive_probs(q, k, scale, causal)
    O = P @ v
    delta = np.sum(np.abs(do) * BF16_U * (np.abs(O) + P @ np.abs(v)), axis=1)
    bq = abs(scale) * delta[:, None] * (P @ np.abs(k))
    bk = abs(scale) * (P * delta[:, None]).T @ np.abs(q)
    return bq, bk
