"""Pins for the list model and the ring interpretation (oracle/listmodel.py).

What pins it (not a retyping of the oracle's own formulas):
* the worked examples printed on the pages (tests/golden/*.json);
* brute force over every small window and history against the one-step
  commutation equation and the three proof goals of [Lean-SWA] §2.4;
* the printed §4.1 identity is shown false on its counterexample, so the
  window comparison is able to see an off-by-one;
* planted bugs (the bug classes listed in [Lean-SWA] §1.2 and the stale
  ``next_position`` of [Prefix-Reuse]) are caught by the window comparison that the GPU
  parity tests use.
"""

import itertools

import pytest

from oracle import listmodel as lm


def cells(n):
    """Symbolic cells: (position, tag)."""
    return [(p, f"kv{p}") for p in range(n)]


def pos_of(c):
    return c[0]


def test_guard_example(golden):
    g = golden("lean_swa_guard_step.json")
    assert lm.step(g["w"], g["cache"], g["kv"]) == g["expected"]


def test_window4_after8_tokens(golden):
    g = golden("prefix_reuse_window4_after8.json")
    hist = cells(g["tokens"])
    win = lm.run(g["w"], hist)
    assert [pos_of(c) for c in win] == g["expected_window_positions"]
    assert lm.window_positions(g["w"], g["tokens"] - 1) == g["expected_window_positions"]
    ring = lm.ring_state(g["w"], hist, pos_of, None)
    assert [pos_of(c) for c in ring] == g["expected_slot_positions"]
    assert lm.ring_to_list(g["w"], ring, g["tokens"]) == win


def test_printed_identity_is_false_and_corrected_form_holds(golden):
    g = golden("lean_swa_drop_identity.json")
    lhs, rhs = lm.printed_drop_identity(g["xs"], g["kv"], g["w"])
    assert lhs == g["printed_lhs"] and rhs == g["printed_rhs"] and lhs != rhs
    lhs2, rhs2 = lm.corrected_drop_identity(g["xs"], g["kv"], g["w"])
    assert lhs2 == rhs2 == g["corrected_rhs"]


@pytest.mark.parametrize("w", range(1, 7))
def test_brute_force_list_model(w):
    """Every history of length 0..4W: run is Valid (§4.2), length <= W (§2.4 goal
    1), positions contiguous and ending at the newest (goal 3), the one-step
    equation (§2.4) holds, the corrected identity holds and the printed one
    fails exactly where the page's premise 1 <= w <= |xs| holds."""
    for n in range(0, 4 * w + 1):
        hist = cells(n)
        c = lm.run(w, hist)
        assert lm.valid(w, hist, c)
        assert len(c) == min(w, n) <= w
        assert lm.position_invariant(c, pos_of)
        if n:
            assert [pos_of(x) for x in c] == lm.window_positions(w, n - 1)
        kv = (n, f"kv{n}")
        assert lm.last_window(w, hist + [kv]) == lm.step(w, lm.last_window(w, hist), kv)
        if 1 <= w <= n:
            lhs, rhs = lm.corrected_drop_identity(hist, kv, w)
            assert lhs == rhs
            assert lhs == lm.last_window(w, hist + [kv])
            plhs, prhs = lm.printed_drop_identity(hist, kv, w)
            assert plhs != prhs and len(prhs) == len(plhs) + 1


@pytest.mark.parametrize("w", range(1, 7))
def test_ring_readback_equals_last_window(w):
    """Two-level check of [Lean-SWA] §3.4: the ring read back through the
    (corrected) ringToList equals the list model after every append, through
    the unfilled, exactly-full, first-overwrite and wrapping phases."""
    for n in range(0, 4 * w + 1):
        hist = cells(n)
        ring = lm.ring_state(w, hist, pos_of, None)
        assert lm.ring_to_list(w, ring, n) == lm.last_window(w, hist)


def test_printed_ring_to_list_reads_garbage_when_unfilled():
    """The page's own warning ([Lean-SWA] §5.1): mapping all w slots reads
    never-written slots before the window fills."""
    w, n = 4, 2
    ring = lm.ring_state(w, cells(n), pos_of, None)
    printed = [ring[(0 + i) % w] for i in range(w)]
    assert None in printed
    assert None not in lm.ring_to_list(w, ring, n)


# ---- planted bugs: the window comparison used by the parity tests must reject each ----

def window_matches(w, ring, n, hist):
    return lm.ring_to_list(w, ring, n) == lm.last_window(w, hist)


def buggy_ring(w, hist, slot_fn):
    buf = [None] * w
    for c in hist:
        buf[slot_fn(pos_of(c))] = c
    return buf


@pytest.mark.parametrize("bug", ["slot_off_by_one", "advance_before_write", "unfilled_base",
                                 "stale_next_position"])
def test_window_comparison_rejects_planted_bugs(bug):
    """[Lean-SWA] §1.2 lists the real bug classes (window offset by one, wrong
    base while unfilled, wrong absolute position, head/tail update order);
    [Prefix-Reuse] plants a stale next_position.  Each must fail the check at
    some phase of a W=4, 12-token run."""
    w = 4
    caught = False
    for n in range(1, 13):
        hist = cells(n)
        if bug == "slot_off_by_one":
            ring = buggy_ring(w, hist, lambda p: (p + 1) % w)
            ok = window_matches(w, ring, n, hist)
        elif bug == "advance_before_write":
            # once the ring is full, the head (oldest slot) is advanced before the
            # overwrite, so the read-back starts one slot late
            ring = lm.ring_state(w, hist, pos_of, None)
            ln = min(w, n)
            start = n - ln + (1 if n > w else 0)
            readback = [ring[(start + i) % w] for i in range(ln)]
            ok = readback == lm.last_window(w, hist)
        elif bug == "unfilled_base":
            ring = lm.ring_state(w, hist, pos_of, None)
            start = n - w  # base taken as n - W even while unfilled
            readback = [ring[(start + i) % w] for i in range(min(w, n))]
            ok = readback == lm.last_window(w, hist)
        else:  # stale next_position: positions restart 2 too late
            shifted = [(p + 2, t) for p, t in hist]
            ring = lm.ring_state(w, shifted, pos_of, None)
            ok = window_matches(w, ring, n, hist)
        if not ok:
            caught = True
    assert caught, bug


def test_position_invariant_rejects_gap():
    assert lm.position_invariant([(3, "a"), (4, "b"), (5, "c")], pos_of)
    assert not lm.position_invariant([(0, "a"), (1, "b"), (3, "c")], pos_of)


def test_exhaustive_small_histories_against_definition():
    """lastWindow against its plain-language definition ([Lean-SWA] §2.2: the
    cache is the most recent W tokens), written as a set comprehension."""
    for w, n in itertools.product(range(1, 6), range(0, 12)):
        hist = cells(n)
        expect = [c for c in hist if pos_of(c) > n - 1 - w]
        assert lm.last_window(w, hist) == expect


def test_no_token_means_no_window():
    """Before the first token (p < 0) the query window is empty."""
    for w in (1, 4, 7):
        assert lm.window_positions(w, -1) == []
        assert lm.window_positions(w, 0) == [0]


def test_valid_compares_contents_not_lengths():
    """Valid (the cache equals lastWindow) fails for a state of the right
    length that holds the wrong cells or the right cells in the wrong order."""
    hist = list(range(10))
    assert lm.valid(4, hist, [6, 7, 8, 9])
    assert not lm.valid(4, hist, [9, 8, 7, 6])
    assert not lm.valid(4, hist, [5, 6, 7, 8])
    assert not lm.valid(4, hist, [6, 7, 8])
