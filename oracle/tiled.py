"""Tiled online-softmax attention in float64 on the CPU.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  This is the second,
independent CPU implementation.  It pins the plain-definition oracle in
``oracle/attention.py``: the two must agree to float64 rounding, and this
module's counters must reproduce the tile, FLOP and traffic tables the source
pages print.

How it is organised (derived from the equations, not from any printed loop):

* The score matrix is cut into a grid of (query block, key block) tiles.
  ``_tile_plan`` classifies every tile before anything is computed: a tile
  whose first key comes after its last query is *skipped* under causal
  masking, a tile that straddles the diagonal is *masked*, every other tile is
  *full* ("LLM Architecture Refresh [3]: Flash Attention Is Exact, and Here's
  the Proof", section 7: only diagonal tiles need a mask, tiles wholly in the
  future are never computed).
* Every query row keeps a notebook (``_RowNotebook``): a reference exponent m,
  the mass l = sum exp(s - m) of the keys seen so far, and the unnormalised
  output u = sum exp(s - m) v.  A computed tile is first summarised on its own
  -- its local max, its local mass and its local unnormalised output, all
  measured against that local max -- and the summary then joins the notebook
  as one composite newcomer: m' = max(m, m~), and both parties are converted
  to m' by the factors exp(m - m') and exp(m~ - m') before they are added
  ("Flash Attention, From First Principles", "The scaffold"; "FlashAttention
  from scratch", Step 2).  A party whose reference is still -inf (nothing
  visible yet) weighs nothing: the guard of "FlashAttention from scratch",
  "Trade-offs and edge cases", against exp(-inf - (-inf)) = NaN.
* The output is u / l, divided once after the last key block ("FlashAttention
  from scratch", Step 3: deferring the division is exact); the saved
  statistic is lse = m + log l (same page, Follow-up questions).
* The single-row normaliser of "LLM Architecture Refresh [3]", section 2, is
  the same notebook with no output column: ``online_normaliser`` folds the
  blocks of one row into (m, l) and records every conversion.
* The recomputing backward ("FlashAttention from scratch", Follow-up
  questions): P = exp(S - L) rebuilt per tile from the saved L;
  dV += P^T dO; dP = dO V^T; D = rowsum(dO * O); dS = P * (dP - D);
  dQ += s dS K; dK += s dS^T Q.
* Counters, worked out from what a tile touches (they reproduce the tables of
  "LLM Architecture Refresh [3]", sections 7 and 8): each computed tile runs
  two products (scores and the value blend) of rows x cols x d multiply-adds,
  two FLOPs each; it streams its key block and its value block from memory;
  each query block reads its queries and writes its output once.  Skipped
  tiles touch nothing.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SKIPPED, MASKED, FULL = "skipped", "masked", "full"


def _tile_kind(causal: bool, q_first: int, q_last: int, k_first: int, k_last: int) -> str:
    """Kind of the tile covering queries q_first..q_last and keys
    k_first..k_last (inclusive), with key j visible to query i iff j <= i."""
    if not causal or k_last <= q_first:
        return FULL
    if k_first > q_last:
        return SKIPPED
    return MASKED


def _spans(n: int, block: int):
    """Inclusive (first, last) index pairs of consecutive blocks; the last one
    may be shorter (a ragged edge)."""
    return [(s, min(s + block, n) - 1) for s in range(0, n, block)]


def _tile_plan(n_q: int, n_k: int, block_q: int, block_k: int, causal: bool):
    """[(query span, [(key span, kind), ...]), ...] for the whole grid."""
    return [((qa, qb), [((ka, kb), _tile_kind(causal, qa, qb, ka, kb))
                        for ka, kb in _spans(n_k, block_k)])
            for qa, qb in _spans(n_q, block_q)]


def causal_tile_counts(n: int, block: int):
    """(computed, skipped) tile counts for an n x n causal score matrix cut
    into square blocks, from the tile classification (no closed form)."""
    kinds = [kind for _, row in _tile_plan(n, n, block, block, True) for _, kind in row]
    skipped = sum(1 for kind in kinds if kind == SKIPPED)
    return len(kinds) - skipped, skipped


def _weight(ref, target):
    """exp(ref - target), with a party at reference -inf weighing 0."""
    ref = np.asarray(ref, dtype=np.float64)
    finite = np.isfinite(ref)
    with np.errstate(invalid="ignore"):
        diff = np.where(finite, ref - target, 0.0)
    return np.where(finite, np.exp(diff), 0.0)


@dataclass
class _RowNotebook:
    """Running state of a set of query rows: reference m [..., r, 1], mass l
    [..., r, 1] and unnormalised output u [..., r, dv], all measured against m."""
    m: np.ndarray
    l: np.ndarray
    u: np.ndarray

    @classmethod
    def empty(cls, lead, rows, dv):
        return cls(np.full((*lead, rows, 1), -np.inf), np.zeros((*lead, rows, 1)),
                   np.zeros((*lead, rows, dv)))

    def admit(self, scores, values, rebase_history: bool = True):
        """Merge one tile (scores [..., r, c], values [..., c, dv]) as a
        composite newcomer: summarise it against its own max, then convert
        both the history and the newcomer to the larger reference."""
        m_tile = np.max(scores, axis=-1, keepdims=True)
        e = _weight(scores, m_tile)              # exp(s - m~), 0 where masked
        l_tile = np.sum(e, axis=-1, keepdims=True)
        u_tile = e @ values
        m_next = np.maximum(self.m, m_tile)
        keep = _weight(self.m, m_next) if rebase_history else np.ones_like(self.m)
        join = _weight(m_tile, m_next)
        self.l = keep * self.l + join * l_tile
        self.u = keep * self.u + join * u_tile
        self.m = m_next
        return keep


def online_normaliser(x, block: int):
    """Stream a 1-D row of logits in blocks; return (m, l, trace).

    Each block is summarised by its own max and mass and merged into the row's
    (m, l) by the conversion law ("LLM Architecture Refresh [3]", section 2;
    "Flash Attention, From First Principles", "The scaffold").  ``trace``
    holds one dict per block: m_old, m_new, correction = exp(m_old - m_new)
    (1 while nothing has been seen), the rebased history l_old * correction,
    and l after the block.
    """
    row = np.asarray(x, dtype=np.float64)
    book = _RowNotebook.empty((), 1, 0)
    trace = []
    for first, last in _spans(row.shape[0], block):
        m_old, l_old = float(book.m[0, 0]), float(book.l[0, 0])
        keep = book.admit(row[None, first:last + 1], np.zeros((last + 1 - first, 0)))
        correction = float(keep[0, 0]) if np.isfinite(m_old) else 1.0
        trace.append(dict(m_old=m_old, m_new=float(book.m[0, 0]), correction=correction,
                          rebased=l_old * correction, l=float(book.l[0, 0])))
    return float(book.m[0, 0]), float(book.l[0, 0]), trace


def _as_bhnd(x):
    a = np.asarray(x, dtype=np.float64)
    if a.ndim == 2:
        a = a[None, None]
    elif a.ndim == 3:
        a = a[None]
    return a


def _masked_scores(q_blk, k_blk, scale, kind, q_first, k_first):
    s = scale * (q_blk @ np.swapaxes(k_blk, -1, -2))
    if kind == MASKED:
        qpos = np.arange(q_first, q_first + q_blk.shape[-2])[:, None]
        kpos = np.arange(k_first, k_first + k_blk.shape[-2])[None, :]
        s = np.where(kpos <= qpos, s, -np.inf)
    return s


def tiled_fwd(q, k, v, scale: float, causal: bool = False,
              block_q: int = 128, block_k: int = 128, elem_bytes: int = 4,
              trace=None, _no_rescale: bool = False):
    """Tiled exact attention with online softmax and one deferred division.

    q, k, v: [B, H, N, d] (2-D or 3-D inputs get leading unit dims).  Returns
    (O, lse, counters) with O [B, H, N, d], lse [B, H, N] (natural log, scaled
    scores) and counters {tiles_computed, blocks_skipped, matmul_flops,
    hbm_bytes}.  ``elem_bytes`` is only used by the traffic counter.

    If ``trace`` is a list, a snapshot dict(q0, k0, m, l, acc) of the query
    block's notebook (acc = the unnormalised output) is appended after every
    computed tile (for the worked examples).

    ``_no_rescale`` plants the classic bug -- the history is never converted
    when the reference moves -- so a test can show the worked-example pin
    catches it.
    """
    q, k, v = _as_bhnd(q), _as_bhnd(k), _as_bhnd(v)
    scale = float(scale)
    lead = q.shape[:2]
    bh = lead[0] * lead[1]
    n, d = q.shape[2], q.shape[3]
    dv = v.shape[-1]
    out = np.empty((*lead, n, dv))
    lse = np.empty((*lead, n))
    counters = dict(tiles_computed=0, blocks_skipped=0, matmul_flops=0, hbm_bytes=0)
    for (qa, qb), row_tiles in _tile_plan(n, k.shape[2], block_q, block_k, causal):
        rows = qb + 1 - qa
        q_blk = q[:, :, qa:qb + 1]
        book = _RowNotebook.empty(lead, rows, dv)
        counters["hbm_bytes"] += bh * (rows * d + rows * dv) * elem_bytes   # Q in, O out
        for (ka, kb), kind in row_tiles:
            if kind == SKIPPED:
                counters["blocks_skipped"] += 1
                continue
            cols = kb + 1 - ka
            counters["tiles_computed"] += 1
            counters["matmul_flops"] += bh * 2 * (rows * cols * d + rows * cols * dv)
            counters["hbm_bytes"] += bh * (cols * d + cols * dv) * elem_bytes  # K, V in
            s = _masked_scores(q_blk, k[:, :, ka:kb + 1], scale, kind, qa, ka)
            book.admit(s, v[:, :, ka:kb + 1], rebase_history=not _no_rescale)
            if trace is not None:
                trace.append(dict(q0=qa, k0=ka, m=book.m.copy(), l=book.l.copy(),
                                  acc=book.u.copy()))
        out[:, :, qa:qb + 1] = book.u / book.l
        lse[:, :, qa:qb + 1] = (book.m + np.log(book.l))[..., 0]
    return out, lse, counters


def tiled_bwd(q, k, v, o, lse, do, scale: float, causal: bool = False,
              block_q: int = 128, block_k: int = 128):
    """Recomputing backward: (dQ, dK, dV) from Q, K, V, O, lse and dO.

    Key blocks on the outside (dK, dV of a key block are complete when its
    column of tiles is done), query blocks inside (dQ gathers a contribution
    from every key block).  Skipped tiles contribute nothing; masked tiles
    rebuild P = 0 for the future keys.  All arrays [B, H, N, d]; lse [B, H, N].
    """
    q, k, v, o, do = (_as_bhnd(x) for x in (q, k, v, o, do))
    lse = np.asarray(lse, dtype=np.float64).reshape(q.shape[:3])
    scale = float(scale)
    n = q.shape[2]
    delta = np.sum(do * o, axis=-1)[..., None]                  # D = rowsum(dO * O)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    plan = _tile_plan(n, k.shape[2], block_q, block_k, causal)
    for kcol, (ka, kb) in enumerate(_spans(k.shape[2], block_k)):
        k_blk, v_blk = k[:, :, ka:kb + 1], v[:, :, ka:kb + 1]
        for (qa, qb), row_tiles in plan:
            kind = row_tiles[kcol][1]
            if kind == SKIPPED:
                continue
            q_blk, do_blk = q[:, :, qa:qb + 1], do[:, :, qa:qb + 1]
            s = _masked_scores(q_blk, k_blk, scale, kind, qa, ka)
            p = np.exp(s - lse[:, :, qa:qb + 1, None])              # P = exp(S - L)
            dp = do_blk @ np.swapaxes(v_blk, -1, -2)
            ds = p * (dp - delta[:, :, qa:qb + 1])
            dv[:, :, ka:kb + 1] += np.swapaxes(p, -1, -2) @ do_blk
            dk[:, :, ka:kb + 1] += scale * (np.swapaxes(ds, -1, -2) @ q_blk)
            dq[:, :, qa:qb + 1] += scale * (ds @ k_blk)
    return dq, dk, dv
