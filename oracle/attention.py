"""Plain-definition attention in float64 on the CPU (the oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  The product path must
never import this module.

What is computed follows the definition the three source pages share:

* "Flash Attention, From First Principles", section "What is attention?":
  O = softmax(Q K^T) V, with the 1/sqrt(d) factor applied to the scores before
  the softmax (the page drops it for the derivation and notes the code applies
  it).  Here the factor is an explicit ``scale`` argument.
* same page, "Stop 2.5: don't set the machine on fire": subtract the row max
  before exponentiating; shift invariance makes that exact.
* same page, "Stop 3: the pour": row i of O is the P-weighted blend of V rows.
* "LLM Architecture Refresh [3]: Flash Attention Is Exact, and Here's the
  Proof", section 5: causal masking forces scores above the diagonal to -inf
  before the softmax, so key j is visible to query i iff j <= i.
* "FlashAttention from scratch", Follow-up questions: the saved statistic is
  the log-sum-exp L = m + log(l), natural log, in scaled-score units.

The backward is the softmax Jacobian written out (not the kernel's D shortcut):
dV = P^T dO and the matmul rule dA = dC B^T, dB = A^T dC ("Flash Attention, From
First Principles", "The ghost at the door"); dP = dO V^T;
dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik); dQ = s dS K, dK = s dS^T Q, the scale
factor s multiplying both ("FlashAttention from scratch", Follow-up questions).

To bound memory the score matrix is formed ``row_chunk`` query rows at a time;
each row's arithmetic is unchanged by that (softmax is row-wise).  For the same
reason ``naive_fwd_rows`` and ``naive_bwd_rows`` evaluate the definitions for
selected rows only (checks at sizes where the whole score matrix is out of
reach); both are pinned against the full forms and torch's float64 autograd.
"""

from __future__ import annotations

import numpy as np

_DEFAULT_ROW_CHUNK = 256


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    return a


def softmax_rows(s) -> np.ndarray:
    """Row-wise softmax with the max subtracted first.

    "Flash Attention, From First Principles", "Stop 2: from scores to
    proportions" (exponentiate, then divide by the sum) and "Stop 2.5"
    (subtract the row max; shift invariance licenses it).  Rows that are
    entirely -inf return all zeros (a row with nothing visible has no mass).
    """
    s = _as_f64(s)
    m = np.max(s, axis=-1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    den = np.sum(e, axis=-1, keepdims=True)
    den_safe = np.where(den > 0, den, 1.0)
    return e / den_safe


def visible_mask(n_q: int, n_k: int, causal: bool, row0: int = 0) -> np.ndarray:
    """Boolean [rows, n_k] mask of visible keys for query rows row0..row0+n_q-1.

    Causal rule ("LLM Architecture Refresh [3]", sections 5 and 7): key j is
    visible to query i iff j <= i.  Non-causal: every key is visible.
    """
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    i = np.arange(row0, row0 + n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i


def _scores(q_rows, k, scale, causal, row0):
    s = scale * (q_rows @ k.T)
    if causal:
        mask = visible_mask(q_rows.shape[0], k.shape[0], True, row0)
        s = np.where(mask, s, -np.inf)
    return s


def naive_probs(q, k, scale: float, causal: bool = False) -> np.ndarray:
    """The full probability matrix P = softmax(scale * Q K^T) for one head.

    Small inputs only (materialises N x N).  q: [N, d], k: [N, d].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    return softmax_rows(_scores(q, k, float(scale), causal, 0))


def _fwd_head(q, k, v, scale, causal, row_chunk):
    n, d = q.shape
    o = np.empty((n, v.shape[1]), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        s = _scores(q[r0:r1], k, scale, causal, r0)          # S = s Q K^T, masked
        m = np.max(s, axis=1, keepdims=True)                  # row max
        e = np.exp(s - m)                                     # shifted exponentials
        l = np.sum(e, axis=1, keepdims=True)                  # row sum
        p = e / l                                             # softmax
        o[r0:r1] = p @ v                                      # the pour
        lse[r0:r1] = (m + np.log(l))[:, 0]                    # L = m + log l
    return o, lse


def naive_fwd(q, k, v, scale: float, causal: bool = False,
              row_chunk: int = _DEFAULT_ROW_CHUNK):
    """Exact attention forward.  Returns (O, lse) in float64.

    q, k, v: arrays of shape [..., N, d] (any leading batch/head dims; q and k
    share N and d, v shares N).  ``scale`` multiplies Q K^T before the softmax.
    lse has shape [..., N].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    scale = float(scale)
    lead = q.shape[:-2]
    n = q.shape[-2]
    o = np.empty(lead + (n, v.shape[-1]), dtype=np.float64)
    lse = np.empty(lead + (n,), dtype=np.float64)
    if n == 0:
        return o, lse
    for idx in np.ndindex(*lead):
        o[idx], lse[idx] = _fwd_head(q[idx], k[idx], v[idx], scale, causal,
                                     row_chunk)
    return o, lse


def naive_fwd_rows(q_rows, k, v, scale: float, causal: bool, positions):
    """Exact attention for selected query rows of one head (sampled checks).

    q_rows: [R, d] queries sitting at sequence positions ``positions`` (R ints);
    k, v: [N, d] the head's full keys and values.  Returns (O [R, d], lse [R]).
    Same definition as ``naive_fwd``; the causal rule uses each row's position.
    """
    q_rows = _as_f64(q_rows)
    k = _as_f64(k)
    v = _as_f64(v)
    pos = np.asarray(positions, dtype=np.int64)
    s = float(scale) * (q_rows @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= pos[:, None], s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    l = np.sum(e, axis=1, keepdims=True)
    return (e / l) @ v, (m + np.log(l))[:, 0]


def _bwd_head(q, k, v, do, scale, causal, row_chunk):
    n = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        s = _scores(q[r0:r1], k, scale, causal, r0)
        p = softmax_rows(s)                                   # P, masked entries 0
        dv += p.T @ do[r0:r1]                                 # dV = P^T dO
        dp = do[r0:r1] @ v.T                                  # dP = dO V^T
        # softmax Jacobian: dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dq[r0:r1] = scale * (ds @ k)                          # dQ = s dS K
        dk += scale * (ds.T @ q[r0:r1])                       # dK = s dS^T Q
    return dq, dk, dv


def naive_bwd(q, k, v, do, scale: float, causal: bool = False,
              row_chunk: int = _DEFAULT_ROW_CHUNK):
    """Gradients (dQ, dK, dV) of sum(O * dO) for O = naive_fwd(q, k, v).

    Shapes as ``naive_fwd``; ``do`` has O's shape.  float64 throughout.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    scale = float(scale)
    lead = q.shape[:-2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    if q.shape[-2] == 0:
        return dq, dk, dv
    for idx in np.ndindex(*lead):
        dq[idx], dk[idx], dv[idx] = _bwd_head(q[idx], k[idx], v[idx], do[idx],
                                              scale, causal, row_chunk)
    return dq, dk, dv



def naive_bwd_rows(q_rows, k, v, do_rows, scale: float, causal: bool, positions,
                   keys=None):
    """What selected query rows of one head carry into the gradients (sampled checks).

    q_rows, do_rows: [R, d] queries and output gradients at sequence positions
    ``positions`` (R distinct ints); k, v: [N, d] the head's full keys and
    values; ``keys``: the key indices whose contributions are returned (all by
    default).  Returns (dQ [R, d] of those rows, their part of dK and of dV
    [len(keys), d]).  Same definition as ``naive_bwd`` (the softmax Jacobian,
    "FlashAttention from scratch", Follow-up questions), restricted to the
    given rows: dQ of a row needs only that row, and dK, dV are sums over
    rows, so for keys that only the given rows see (under causal masking, the
    last keys of the sequence when the rows are the last positions) the parts
    returned are those keys' whole gradients.
    """
    q_rows = _as_f64(q_rows)
    k = _as_f64(k)
    v = _as_f64(v)
    do_rows = _as_f64(do_rows)
    scale = float(scale)
    pos = np.asarray(positions, dtype=np.int64)
    s = scale * (q_rows @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= pos[:, None], s, -np.inf)
    p = softmax_rows(s)
    dp = do_rows @ v.T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    sel = np.arange(k.shape[0]) if keys is None else np.asarray(keys, dtype=np.int64)
    return scale * (ds @ k), scale * (ds[:, sel].T @ q_rows), p[:, sel].T @ do_rows

# ---------------------------------------------------------------------------
# Grouped-query attention
#
# The pages name multi-query and grouped-query attention as the fix for the
# key/value cache ("LLM Architecture Refresh [3]", section 6, the table that
# sets the KV cache against the score matrix; "Flash Attention, From First
# Principles", "Honesty time", item 6) without defining them further.  The
# reading taken: H query heads share Hkv key/value heads, H a multiple of Hkv,
# and query head h uses key/value head h // (H // Hkv) (consecutive query
# heads form a group).  Per query head the operation is exactly the one above.
# ---------------------------------------------------------------------------

def kv_head_of(h: int, H: int, Hkv: int) -> int:
    """Key/value head serving query head h (groups of H // Hkv consecutive heads)."""
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"H={H} is not a multiple of Hkv={Hkv}")
    return h // (H // Hkv)


def naive_fwd_gqa(q, k, v, scale: float, causal: bool = False,
                  row_chunk: int = _DEFAULT_ROW_CHUNK):
    """Exact attention with shared key/value heads.  Returns (O, lse), float64.

    q: [B, H, N, d]; k, v: [B, Hkv, N, d].  Query head h attends with
    key/value head kv_head_of(h, H, Hkv).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, n, _ = q.shape
    Hkv = k.shape[1]
    o = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    if n == 0:
        return o, lse
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            o[b, h], lse[b, h] = _fwd_head(q[b, h], k[b, g], v[b, g], float(scale),
                                           causal, row_chunk)
    return o, lse


def naive_bwd_gqa(q, k, v, do, scale: float, causal: bool = False,
                  row_chunk: int = _DEFAULT_ROW_CHUNK):
    """Gradients of sum(O * dO) for O = naive_fwd_gqa(q, k, v).

    A shared key/value head receives the sum of the gradients of every query
    head that reads it (the chain rule through a shared input).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, H, n, _ = q.shape
    Hkv = k.shape[1]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if n == 0:
        return dq, dk, dv
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            dq[b, h], dk_h, dv_h = _bwd_head(q[b, h], k[b, g], v[b, g], do[b, h],
                                             float(scale), causal, row_chunk)
            dk[b, g] += dk_h
            dv[b, g] += dv_h
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Queries and keys of different lengths (cross-attention, decode against a
# key/value cache)
#
# The pages treat one length n for queries and keys ("LLM Architecture
# Refresh [3]", the notes before the references: one forward pass over n
# tokens, so the score matrix is square) and note that generation splits a
# sequence into a prompt and generated tokens.  The reading taken for Nq query
# rows against Nk keys: the queries are the LAST Nq positions of the
# sequence, so with causal masking query i (0-based) sees key j iff
# j <= i + (Nk - Nq) (bottom-right alignment; for Nq = Nk this is the j <= i
# rule of section 5).  A query with no visible key (only possible when
# Nq > Nk) has no probability mass: its output row is 0 and its log-sum-exp
# is -inf, the identity of the block-merge law ("Flash Attention, From First
# Principles", "The scaffold").
# ---------------------------------------------------------------------------

def visible_mask_kv(n_q: int, n_k: int, causal: bool) -> np.ndarray:
    """Boolean [n_q, n_k] mask: key j visible to query i (bottom-right causal)."""
    if not causal:
        return np.ones((n_q, n_k), dtype=bool)
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i + (n_k - n_q)


def naive_fwd_kv(q, k, v, scale: float, causal: bool = False):
    """Exact attention of Nq queries against Nk keys.  Returns (O, lse), float64.

    q: [B, H, Nq, d]; k, v: [B, Hkv, Nk, d] with H a multiple of Hkv (query
    head h reads key/value head h // (H // Hkv)).  Rows without a visible key
    give O = 0 and lse = -inf.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, nq, _ = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    o = np.zeros(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.full(q.shape[:-1], -np.inf, dtype=np.float64)
    if nq == 0 or nk == 0:
        return o, lse
    mask = visible_mask_kv(nq, nk, causal)
    live = mask.any(axis=1)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            s = float(scale) * (q[b, h] @ k[b, g].T)             # S = s Q K^T
            s = np.where(mask, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(s - m)                                    # masked -> 0
            l = np.sum(e, axis=1, keepdims=True)
            l_safe = np.where(l > 0, l, 1.0)
            o[b, h] = (e / l_safe) @ v[b, g]
            lse[b, h] = np.where(live, (m + np.log(l_safe))[:, 0], -np.inf)
    return o, lse


def naive_bwd_kv(q, k, v, do, scale: float, causal: bool = False):
    """Gradients of sum(O * dO) for O = naive_fwd_kv(q, k, v).

    The softmax Jacobian per row as in ``naive_bwd``; rows with no visible key
    contribute nothing.  Shared key/value heads sum their query heads' parts.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, H, nq, _ = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if nq == 0 or nk == 0:
        return dq, dk, dv
    mask = visible_mask_kv(nq, nk, causal)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            s = float(scale) * (q[b, h] @ k[b, g].T)
            p = softmax_rows(np.where(mask, s, -np.inf))         # empty rows -> 0
            dv[b, g] += p.T @ do[b, h]                           # dV = P^T dO
            dp = do[b, h] @ v[b, g].T                            # dP = dO V^T
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dq[b, h] = float(scale) * (ds @ k[b, g])             # dQ = s dS K
            dk[b, g] += float(scale) * (ds.T @ q[b, h])          # dK = s dS^T Q
    return dq, dk, dv


# ---------------------------------------------------------------------------
# 8-bit floating-point inputs
#
# "LLM Architecture Refresh [3]", section 8 points at FP8 matrix inputs (the
# FA-3 direction) without fixing a format.  The reading taken: the OCP e4m3
# format ("float8 e4m3fn": 1 sign bit, 4 exponent bits with bias 7, 3
# mantissa bits; exponent 0 holds the subnormals m/8 * 2^-6; the all-ones
# exponent with mantissa 7 is NaN; no infinities), one dequantisation factor
# per tensor.  The oracle decodes the bytes to the exact values they stand for
# and evaluates the plain definition on them in float64.
# ---------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """float64 values of OCP e4m3 byte codes (any integer array)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, mant / 8.0 * 2.0 ** -6, (1.0 + mant / 8.0) * 2.0 ** (e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def naive_fwd_fp8(q8, k8, v8, q_scale: float, k_scale: float, v_scale: float, scale: float,
                  causal: bool = False):
    """Exact attention of the dequantised e4m3 tensors, float64: (O, lse).

    q8, k8, v8: e4m3 byte codes [..., N, d]; the tensors are q_scale * q8,
    k_scale * k8 and v_scale * v8.
    """
    q = float(q_scale) * e4m3_decode(q8)
    k = float(k_scale) * e4m3_decode(k8)
    v = float(v_scale) * e4m3_decode(v8)
    return naive_fwd(q, k, v, scale, causal)
