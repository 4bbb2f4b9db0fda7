"""Tiled online-softmax attention in float64 on the CPU.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  This is the second,
independent CPU implementation.  It pins the plain-definition oracle in
``oracle/attention.py``: the two must agree to float64 rounding, and this
module's counters must reproduce the tile, FLOP and traffic tables the source
pages print.

Steps, in the order the pages give them:

* "LLM Architecture Refresh [3]: Flash Attention Is Exact, and Here's the
  Proof", section 2: the online normaliser -- a running max m and running sum l,
  with the held sum rebased by exp(m_old - m_new) whenever a block raises the
  max.
* same page, section 4: outer loop over query blocks, inner loop streaming
  key/value blocks; the accumulated output is rescaled by the same factor as l
  and divided by l once, after the last block.
* "Flash Attention, From First Principles", "The scaffold": a tile row's local
  max and local sum merge into the notebook by the same law (a composite
  newcomer).
* "LLM Architecture Refresh [3]", section 7: with causal masking a key block
  that starts after the query block's last row is skipped, not computed; only
  tiles that straddle the diagonal need a mask.
* "FlashAttention from scratch", Trade-offs and edge cases: a row whose running
  max is still -inf would give exp(-inf - (-inf)) = NaN; such a row takes
  correction 1 and contributes nothing.
* "FlashAttention from scratch", Follow-up questions: the backward recomputes
  P = exp(S - L) from the saved L = m + log l; dV += P^T dO; dP = dO V^T;
  D = rowsum(dO * O); dS = P * (dP - D); dQ += s dS K; dK += s dS^T Q.
* Counters ("LLM Architecture Refresh [3]", sections 7 and 8): skipped tiles;
  matmul FLOPs 2 * (2 * batch * heads * rows * cols * d) per computed tile;
  traffic 2 * batch * heads * cols * d * elem per computed tile for K and V,
  plus Q read and O written once per query block.
"""

from __future__ import annotations

import numpy as np


def _tile_is_skipped(causal: bool, q0: int, rows: int, k0: int) -> bool:
    """A key block whose first key lies after the query block's last row."""
    return causal and k0 > q0 + rows - 1


def causal_tile_counts(n: int, block: int):
    """(computed, skipped) tile counts of the tiled loop for an n x n causal
    score matrix cut into square blocks.  Runs the loop's own skip predicate
    over every tile; no closed form is used."""
    computed = skipped = 0
    for q0 in range(0, n, block):
        rows = min(block, n - q0)
        for k0 in range(0, n, block):
            if _tile_is_skipped(True, q0, rows, k0):
                skipped += 1
            else:
                computed += 1
    return computed, skipped


def online_normaliser(x, block: int):
    """Stream a 1-D row of logits in blocks; return (m, l, trace).

    "LLM Architecture Refresh [3]", section 2: m_new = max(m_old, max(block));
    l_new = l_old * exp(m_old - m_new) + sum(exp(block - m_new)).
    ``trace`` holds one dict per block: m_old, m_new, correction, the rebased
    history l_old * correction, and l after the block.
    """
    x = np.asarray(x, dtype=np.float64)
    m = -np.inf
    l = 0.0
    trace = []
    for start in range(0, x.shape[0], block):
        blk = x[start:start + block]
        m_new = max(m, float(np.max(blk)))
        correction = 1.0 if m_new == -np.inf else float(np.exp(m - m_new))
        rebased = l * correction
        l = rebased + float(np.sum(np.exp(blk - m_new)))
        trace.append(dict(m_old=m, m_new=m_new, correction=correction,
                          rebased=rebased, l=l))
        m = m_new
    return m, l, trace


def _as_bhnd(x):
    a = np.asarray(x, dtype=np.float64)
    if a.ndim == 2:
        a = a[None, None]
    elif a.ndim == 3:
        a = a[None]
    return a


def tiled_fwd(q, k, v, scale: float, causal: bool = False,
              block_q: int = 128, block_k: int = 128, elem_bytes: int = 4,
              trace=None, _no_rescale: bool = False):
    """Tiled exact attention with online softmax and one deferred division.

    q, k, v: [B, H, N, d] (2-D or 3-D inputs get leading unit dims).  Returns
    (O, lse, counters) with O [B, H, N, d], lse [B, H, N] (natural log, scaled
    scores) and counters {tiles_computed, blocks_skipped, matmul_flops,
    hbm_bytes}.  ``elem_bytes`` is only used by the traffic counter.

    If ``trace`` is a list, a snapshot dict(q0, k0, m, l, acc) of the running
    notebook is appended after every computed tile (for the worked examples).

    ``_no_rescale`` plants the classic bug (history never rebased when the max
    moves) so a test can show the worked-example pin catches it.
    """
    q = _as_bhnd(q)
    k = _as_bhnd(k)
    v = _as_bhnd(v)
    scale = float(scale)
    b, h, n, d = q.shape
    dv_ = v.shape[-1]
    out = np.empty((b, h, n, dv_), dtype=np.float64)
    lse = np.empty((b, h, n), dtype=np.float64)
    counters = dict(tiles_computed=0, blocks_skipped=0, matmul_flops=0,
                    hbm_bytes=0)
    for q0 in range(0, n, block_q):
        qi = q[:, :, q0:q0 + block_q]
        rows = qi.shape[2]
        counters["hbm_bytes"] += 2 * b * h * rows * d * elem_bytes  # Q in, O out
        m = np.full((b, h, rows, 1), -np.inf)
        l = np.zeros((b, h, rows, 1))
        acc = np.zeros((b, h, rows, dv_))
        qpos = np.arange(q0, q0 + rows)
        for k0 in range(0, n, block_k):
            if _tile_is_skipped(causal, q0, rows, k0):
                counters["blocks_skipped"] += 1
                continue
            kj = k[:, :, k0:k0 + block_k]
            vj = v[:, :, k0:k0 + block_k]
            cols = kj.shape[2]
            counters["tiles_computed"] += 1
            counters["matmul_flops"] += 2 * (2 * b * h * rows * cols * d)
            counters["hbm_bytes"] += 2 * b * h * cols * d * elem_bytes
            s = scale * (qi @ np.swapaxes(kj, -1, -2))        # score tile
            if causal and k0 + cols - 1 > q0:                  # straddles diagonal
                kpos = np.arange(k0, k0 + cols)
                s = np.where(kpos[None, :] <= qpos[:, None], s, -np.inf)
            m_tile = np.max(s, axis=-1, keepdims=True)
            m_new = np.maximum(m, m_tile)
            dead = ~np.isfinite(m_new)                         # nothing seen yet
            m_ref = np.where(dead, 0.0, m_new)
            correction = np.where(dead, 1.0, np.exp(m - m_ref))
            if _no_rescale:
                correction = np.ones_like(correction)
            p = np.where(dead, 0.0, np.exp(s - m_ref))
            l = l * correction + np.sum(p, axis=-1, keepdims=True)
            acc = acc * correction + p @ vj                    # rebase, then add
            m = m_new
            if trace is not None:
                trace.append(dict(q0=q0, k0=k0, m=m.copy(), l=l.copy(),
                                  acc=acc.copy()))
        out[:, :, q0:q0 + rows] = acc / l                      # one division
        lse[:, :, q0:q0 + rows] = (m + np.log(l))[..., 0]
    return out, lse, counters


def tiled_bwd(q, k, v, o, lse, do, scale: float, causal: bool = False,
              block_q: int = 128, block_k: int = 128):
    """Recomputing backward: (dQ, dK, dV) from Q, K, V, O, lse and dO.

    Outer loop over key/value blocks (dK, dV accumulate per block), inner loop
    over query blocks (dQ accumulates across key blocks).  Tiles wholly in the
    future are skipped under causal masking.  All arrays [B, H, N, d]; lse
    [B, H, N].
    """
    q = _as_bhnd(q)
    k = _as_bhnd(k)
    v = _as_bhnd(v)
    o = _as_bhnd(o)
    do = _as_bhnd(do)
    lse = np.asarray(lse, dtype=np.float64).reshape(q.shape[:3])
    scale = float(scale)
    n = q.shape[2]
    dmat = np.sum(do * o, axis=-1)                              # D = rowsum(dO*O)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for k0 in range(0, n, block_k):
        kj = k[:, :, k0:k0 + block_k]
        vj = v[:, :, k0:k0 + block_k]
        cols = kj.shape[2]
        kpos = np.arange(k0, k0 + cols)
        for q0 in range(0, n, block_q):
            rows = min(block_q, n - q0)
            if _tile_is_skipped(causal, q0, rows, k0):
                continue
            qi = q[:, :, q0:q0 + rows]
            doi = do[:, :, q0:q0 + rows]
            s = scale * (qi @ np.swapaxes(kj, -1, -2))
            if causal and k0 + cols - 1 > q0:
                qpos = np.arange(q0, q0 + rows)
                s = np.where(kpos[None, :] <= qpos[:, None], s, -np.inf)
            p = np.exp(s - lse[:, :, q0:q0 + rows, None])       # P = exp(S - L)
            dv[:, :, k0:k0 + cols] += np.swapaxes(p, -1, -2) @ doi
            dp = doi @ np.swapaxes(vj, -1, -2)
            ds = p * (dp - dmat[:, :, q0:q0 + rows, None])
            dq[:, :, q0:q0 + rows] += scale * (ds @ kj)
            dk[:, :, k0:k0 + cols] += scale * (np.swapaxes(ds, -1, -2) @ qi)
    return dq, dk, dv
