"""Full-history decoder: what one sequence's cache must hold and produce.

The oracle keeps every appended token with its absolute position (the cache
record of [Prefix-Reuse] "哪些東西必須一起裁剪": K, V, per-row absolute positions
and ``next_position``) and answers each query with the masked full-history
attention of [Lean-SWA] §2.1.  From the same history it derives the state a
fixed ring of ``W`` slots must be in ([Lean-SWA] §3.4) and, for the INT8
cache, the codes, scales, witnesses and the exact staging tokens.

Readings taken:
* Positions are 0-based and contiguous; token ``j`` of a sequence has
  position ``j`` and ``next_position`` is the number of tokens appended.
* A decode step appends first and then attends, so the query of the step at
  position ``t`` sees ``len = min(W, t + 1)`` tokens ``[t - len + 1, t]``.
* Appending ``T`` tokens at once is the same as ``T`` single appends.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from . import attention, int8, listmodel


class SequenceHistory:
    """Every token of one sequence, all heads: ``k``, ``v`` are ``[H, n, D]``."""

    def __init__(self, num_heads: int, head_dim: int):
        self.H = num_heads
        self.D = head_dim
        self._k = []
        self._v = []
        self._n = 0
        self._cache = None

    @property
    def next_position(self) -> int:
        return self._n

    def append(self, k_new: np.ndarray, v_new: np.ndarray) -> None:
        """Append ``T`` tokens ``[H, T, D]`` at positions ``n .. n+T-1``."""
        k_new = np.asarray(k_new, dtype=np.float64)
        v_new = np.asarray(v_new, dtype=np.float64)
        assert k_new.shape == v_new.shape and k_new.shape[0] == self.H
        assert k_new.shape[2] == self.D
        self._k.append(k_new)
        self._v.append(v_new)
        self._n += k_new.shape[1]
        self._cache = None

    def arrays(self):
        """(positions [n], k [H, n, D], v [H, n, D]) as float64."""
        if self._cache is None:
            if self._k:
                k = np.concatenate(self._k, axis=1)
                v = np.concatenate(self._v, axis=1)
            else:
                k = np.zeros((self.H, 0, self.D))
                v = np.zeros((self.H, 0, self.D))
            self._k, self._v = [k], [v]
            self._cache = (np.arange(self._n, dtype=np.int64), k, v)
        return self._cache

    def attend(self, q: np.ndarray, w: int) -> np.ndarray:
        """Masked full-history attention of the query at step ``n - 1``;
        ``q`` is ``[H, D]``, the result ``[H, D]`` float64."""
        pos, k, v = self.arrays()
        t = self._n - 1
        return np.stack([attention.masked_attention(q[h], pos, k[h], v[h], t, w)
                         for h in range(self.H)])

    def attend_window(self, q: np.ndarray, w: int) -> np.ndarray:
        """Attention over ``lastWindow(W, history)`` only (no mask): the
        target semantics of [Lean-SWA] §2.2, used for the theorem check."""
        pos, k, v = self.arrays()
        idx = listmodel.last_window(w, list(range(self._n)))
        return np.stack([attention.plain_attention(q[h], k[h][idx], v[h][idx])
                         for h in range(self.H)])


def expected_ring(positions: np.ndarray, w: int) -> np.ndarray:
    """Per ring slot, the history index (= position) of the cell it holds
    after all appends, or -1 for a never-written slot ([Lean-SWA] §3.4)."""
    idx = listmodel.ring_state(w, list(int(p) for p in positions), lambda p: p, -1)
    return np.asarray(idx, dtype=np.int64)


def expected_int8_store(k: np.ndarray, v: np.ndarray, next_position: int, w: int,
                        band: int = int8.BAND) -> dict:
    """What an INT8 ring of ``w`` slots holds for one (sequence, head).

    ``k``, ``v`` are the ``[n, D]`` history rows (position = row index).  The
    ring holds the complete blocks only: slot ``s`` carries the newest token
    ``j < 16 * (n // 16)`` with ``j mod w == s``.  Returns the slot positions
    (-1 if none), codes, per-slot-block scales, the exact float64 witness
    rows, and the positions that sit in the 16-token staging area (index
    ``pos mod 16``).
    """
    n = next_position
    blk = int8.BLOCK
    nb = n // blk
    ks, kc = int8.quantize_history(np.asarray(k)[: nb * blk], nb)
    vs, vc = int8.quantize_history(np.asarray(v)[: nb * blk], nb)
    slot_pos = expected_ring(np.arange(nb * blk), w)
    d = k.shape[-1]
    k_codes = np.zeros((w, d), dtype=np.int8)
    v_codes = np.zeros((w, d), dtype=np.int8)
    k_scale = np.zeros(w // blk, dtype=np.float32)
    v_scale = np.zeros(w // blk, dtype=np.float32)
    wit = np.zeros((w, d // band), dtype=np.float64)
    for s in range(w):
        j = slot_pos[s]
        if j < 0:
            continue
        k_codes[s] = kc[j]
        v_codes[s] = vc[j]
        k_scale[s // blk] = ks[j // blk]
        v_scale[s // blk] = vs[j // blk]
        r = np.asarray(k[j], dtype=np.float64) - int8.dequantize(kc[j], ks[j // blk])
        wit[s] = int8.band_norms(r, band)
    staged = list(range(nb * blk, n))
    return {
        "slot_pos": slot_pos,
        "k_codes": k_codes,
        "v_codes": v_codes,
        "k_scale": k_scale,
        "v_scale": v_scale,
        "witness": wit,
        "staged_positions": staged,
    }
