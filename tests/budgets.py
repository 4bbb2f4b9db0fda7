"""Error budgets shared by the GPU parity tests (test infrastructure: oracle
quantities only, no GPU result enters a bound)."""

import numpy as np

from oracle import kv_head_of, naive_probs, softmax_rows, visible_mask_kv

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


def d_term_bounds_kv(q, k, v, do, scale, causal):
    """``d_term_bounds`` for grouped heads and different lengths: q, do
    [B, H, Nq, d], k, v [B, Hkv, Nk, d] (query head h reads key/value head
    h // (H // Hkv); the Nq queries are the last positions).  dQ's bound is per
    query head as above; a shared key/value head's dK sums its query heads'
    dS, so its bound sums theirs.  Returns (bound on dQ [B, H, Nq, d], bound on
    dK [B, Hkv, Nk, d])."""
    B, H, nq, _ = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    bq = np.zeros(q.shape)
    bk = np.zeros(k.shape)
    if nq == 0 or nk == 0:
        return bq, bk
    mask = visible_mask_kv(nq, nk, causal)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            s = float(scale) * (q[b, h] @ k[b, g].T)
            P = softmax_rows(np.where(mask, s, -np.inf))
            O = P @ v[b, g]
            delta = np.sum(np.abs(do[b, h]) * BF16_U * (np.abs(O) + P @ np.abs(v[b, g])), axis=1)
            bq[b, h] = abs(scale) * delta[:, None] * (P @ np.abs(k[b, g]))
            bk[b, g] += abs(scale) * (P * delta[:, None]).T @ np.abs(q[b, h])
    return bq, bk
