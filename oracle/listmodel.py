"""List model of the sliding-window KV cache and its ring-buffer interpretation.

Follows [Lean-SWA] §2.3 (``lastWindow``, ``Valid``), §2.4 (the three proof
goals and the one-step commutation equation), §3.2 (``KVCell`` carries an
absolute position; ``PositionInvariant``), §3.3 (``step``), §3.4
(``ringToList``) and §4.1-§4.2 (``run`` as a left fold, the drop/append
identity).  Cells are opaque Python values; a cell's position is read through
the ``pos_of`` callable where a position is needed.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

from typing import Callable, List, Sequence, Tuple, TypeVar

T = TypeVar("T")


def last_window(w: int, hs: Sequence[T]) -> List[T]:
    """[Lean-SWA] §2.3: drop the first ``len(hs) - min(w, len(hs))`` cells."""
    n = len(hs)
    return list(hs[n - min(w, n):])


def valid(w: int, hs: Sequence[T], c: Sequence[T]) -> bool:
    """[Lean-SWA] §2.3: a cache state is valid iff it equals lastWindow."""
    return list(c) == last_window(w, hs)


def step(w: int, c: Sequence[T], kv: T) -> List[T]:
    """[Lean-SWA] §3.3: append, then drop the head if the length exceeds w."""
    c2 = list(c) + [kv]
    if w < len(c2):
        return c2[1:]
    return c2


def run(w: int, tokens: Sequence[T]) -> List[T]:
    """[Lean-SWA] §4.2: ``run`` is the left fold of ``step`` from the empty cache."""
    c: List[T] = []
    for kv in tokens:
        c = step(w, c, kv)
    return c


def position_invariant(c: Sequence[T], pos_of: Callable[[T], int]) -> bool:
    """[Lean-SWA] §3.2: there is a base with ``pos(c[i]) = base + i`` for all i."""
    if not c:
        return True
    base = pos_of(c[0])
    return all(pos_of(cell) == base + i for i, cell in enumerate(c))


def window_positions(w: int, p: int) -> List[int]:
    """Positions the query of step ``p`` sees: [Lean-SWA] §2.4 goal 3.

    The page states the full-window form ``pos_i = t - W + 1 + i``.  Reading
    taken for the unfilled phase (positions are 0-based, so ``p + 1`` tokens
    exist): the window holds ``len = min(W, p + 1)`` cells with
    ``pos_i = p - len + 1 + i``.  Signed arithmetic throughout, never a
    truncating subtraction ([Lean-SWA] §4.3, §5.2).
    """
    if p < 0:
        return []
    ln = min(w, p + 1)
    return [p - ln + 1 + i for i in range(ln)]


def printed_drop_identity(xs: Sequence[T], kv: T, w: int) -> Tuple[List[T], List[T]]:
    """Both sides of the identity as printed in [Lean-SWA] §4.1 / §4.3.

    ``(xs ++ [kv]).drop (|xs| + 1 - w)`` versus ``xs.drop (|xs| - w) ++ [kv]``,
    with Lean's truncating Nat subtraction.  As printed the two sides have
    lengths ``w`` and ``w + 1`` whenever ``1 <= w <= |xs|``, so the identity is
    false there; the tests show this on a concrete counterexample.
    """
    n = len(xs)
    lhs = (list(xs) + [kv])[max(n + 1 - w, 0):]
    rhs = list(xs)[max(n - w, 0):] + [kv]
    return lhs, rhs


def corrected_drop_identity(xs: Sequence[T], kv: T, w: int) -> Tuple[List[T], List[T]]:
    """The form of the §4.1 identity that holds for ``1 <= w <= |xs|``.

    ``(xs ++ [kv]).drop (|xs| + 1 - w) = xs.drop (|xs| + 1 - w) ++ [kv]``: both
    sides keep the last ``w - 1`` old cells and then ``kv``.
    """
    n = len(xs)
    lhs = (list(xs) + [kv])[max(n + 1 - w, 0):]
    rhs = list(xs)[max(n + 1 - w, 0):] + [kv]
    return lhs, rhs


def ring_slot(w: int, pos: int) -> int:
    """[Lean-SWA] §3.4: a fixed array of ``w`` slots; the cell with absolute
    position ``pos`` is written at ``pos mod w``, overwriting the oldest."""
    return pos % w


def ring_to_list(w: int, buf: Sequence[T], next_position: int) -> List[T]:
    """Logical view of a ring of ``w`` slots after ``next_position`` appends.

    [Lean-SWA] §3.4 prints ``(List.range w).map (fun i => buf[(head+i) % w])``,
    which maps all ``w`` slots and so reads never-written slots in the unfilled
    phase (the page's own warning in §5.1).  Reading taken: with
    ``n = next_position``, ``len = min(w, n)``, ``start = n - len`` (the
    oldest live position), element ``i`` is ``buf[(start + i) mod w]``.
    """
    ln = min(w, next_position)
    start = next_position - ln
    return [buf[(start + i) % w] for i in range(ln)]


def ring_state(w: int, tokens: Sequence[T], pos_of: Callable[[T], int], empty: T) -> List[T]:
    """Physical content of the ring after writing ``tokens`` in order.

    Each cell goes to slot ``pos mod w`` ([Lean-SWA] §3.4); slots that were
    never written hold ``empty``.
    """
    buf = [empty] * w
    for cell in tokens:
        buf[ring_slot(w, pos_of(cell))] = cell
    return buf
