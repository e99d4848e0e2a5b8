"""Reference attention in float64.

* ``masked_attention``: the specification of [Lean-SWA] §2.1 -- the whole
  history is kept and logits of positions outside ``[t - W + 1, t]`` are set
  to minus infinity (``mask_window`` plus ``mask_causal``).
* ``plain_attention``: single-query attention over an explicit list of rows,
  as the decode step of [KV-Loop] §三 computes it (scores ``q . K^T / sqrt(d)``,
  max-subtracted softmax, weighted sum of V); [KV-Loop] §三 also notes that a
  single decode query needs no causal mask.

Both return float64.  Reading taken for an empty visible set (the pages are
silent): the output is the zero vector.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax over the last axis ([KV-Loop] §三).  ``-inf``
    entries get weight exactly 0."""
    scores = np.asarray(scores, dtype=np.float64)
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def plain_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """``softmax(q . K^T / sqrt(D)) . V`` for one query over rows ``k``, ``v``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1], dtype=np.float64)
    scores = (k @ q) / np.sqrt(d)
    return softmax_weights(scores) @ v


def visibility(pos: np.ndarray, t: int, w: int) -> np.ndarray:
    """[Lean-SWA] §2.1: position ``j`` is visible to the query of step ``t``
    iff ``t - w + 1 <= j`` (window) and ``j <= t`` (causal)."""
    pos = np.asarray(pos, dtype=np.int64)
    return (pos >= t - w + 1) & (pos <= t)


def masked_attention(q: np.ndarray, pos: np.ndarray, k: np.ndarray, v: np.ndarray,
                     t: int, w: int) -> np.ndarray:
    """[Lean-SWA] §2.1 reference semantics over the FULL history.

    ``pos[j]`` is the absolute position of history row ``j``; ``k``, ``v`` are
    ``[n, D]``.  Logits of invisible rows are ``-inf`` before the softmax.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    vis = visibility(pos, t, w)
    if not np.any(vis):
        return np.zeros(v.shape[-1], dtype=np.float64)
    d = q.shape[-1]
    scores = np.where(vis, (k @ q) / np.sqrt(d), -np.inf)
    return softmax_weights(scores) @ v
