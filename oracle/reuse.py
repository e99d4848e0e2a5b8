"""Prefix reuse: truncating a cache to a common prefix, or falling back.

[Prefix-Reuse]:
* "先看一次歷史編輯": the reusable part of a cache for a new request is the
  leading run of tokens equal to the cached ones (not every position whose
  token happens to match);
* "哪些東西必須一起裁剪": keep K, V and the positions of the first ``cut`` rows
  and continue from ``next_position = cut``;
* "查詢流程與快取所有權": the cut is at most ``len(query) - 1`` so the last
  token is always recomputed;
* "為什麼滑窗部分命中必須回退": a window cache no longer holds evicted rows, so
  a partial hit on it must fall back to recomputation.

Reading taken for the ring: truncating to ``cut`` is exact iff every row of
``lastWindow(W, history[:cut])`` is still stored in the form the cache keeps
it.  For rows that holds when ``0 <= cut <= n`` and nothing was evicted yet
(``n <= W``), nothing is dropped (``cut == n``), or nothing is kept
(``cut == 0``, a reset).  The INT8 cache
also needs the cut on a block boundary or inside the exact staging tail
(``cut >= 16 * (n // 16)``): a committed block keeps only codes, so its first
rows cannot go back to exact staging rows.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

from typing import Sequence


def common_prefix(old: Sequence[int], new: Sequence[int]) -> int:
    """Length of the leading run where ``old`` and ``new`` agree, capped at
    ``len(new) - 1`` so the newest token is always recomputed."""
    n = 0
    for a, b in zip(old, new):
        if a != b:
            break
        n += 1
    return max(0, min(n, len(new) - 1))


def truncation_exact(n: int, cut: int, w: int, int8: bool = False) -> bool:
    """Whether a ring of ``w`` slots after ``n`` appends can be truncated to
    ``cut`` without recomputing anything (see the module docstring)."""
    if cut < 0 or cut > n:
        return False
    if n > w and cut not in (0, n):
        return False
    if int8 and cut % 16 != 0 and cut < 16 * (n // 16):
        return False
    return True
