"""Pins for prefix reuse (oracle/reuse.py): the page's edit example and its
window fallback example, and brute force of the truncation rule against the
list model (truncation is exact iff the window of the shorter history is a
sub-list of what the ring still stores)."""

import pytest

from oracle import listmodel, reuse


def test_edit_example(golden):
    g = golden("prefix_reuse_edit_example.json")
    assert reuse.common_prefix(g["old"], g["new"]) == g["expected_cut"]


def test_cut_keeps_last_token():
    assert reuse.common_prefix([1, 2, 3], [1, 2, 3]) == 2
    assert reuse.common_prefix([1, 2, 3], [1]) == 0
    assert reuse.common_prefix([5], [6, 7]) == 0


def test_window_fallback_example(golden):
    g = golden("prefix_reuse_window_fallback.json")
    n, cut = g["tokens"], g["cut"]
    assert reuse.truncation_exact(n, cut, g["full_cache_capacity"]) is g["expected_full_cache_reusable"]
    assert reuse.truncation_exact(n, cut, g["window"]) is g["expected_window_reusable"]


@pytest.mark.parametrize("w", range(1, 8))
def test_rule_matches_list_model(w):
    """Rows: exact iff every position of lastWindow(W, hist[:cut]) is among the
    positions the ring holds after n appends."""
    for n in range(0, 4 * w + 2):
        held = set(listmodel.last_window(w, list(range(n))))
        for cut in range(-1, n + 2):
            if 0 <= cut <= n:
                need = set(listmodel.last_window(w, list(range(cut))))
                expect = need <= held
            else:
                expect = False
            assert reuse.truncation_exact(n, cut, w) == expect, (w, n, cut)


def test_int8_rule_matches_block_model():
    """INT8: rows of committed blocks are codes; a cut inside a committed block
    would need its leading rows exact again, so it must fall back."""
    w = 64
    for n in range(0, 140):
        for cut in range(0, n + 1):
            rows_ok = reuse.truncation_exact(n, cut, w)
            committed_tail = (cut % 16 != 0) and (cut < 16 * (n // 16))
            assert reuse.truncation_exact(n, cut, w, int8=True) == (rows_ok and not committed_tail)


def test_empty_query_reuses_nothing():
    """An empty new request has no token to recompute and reuses nothing: the
    cut is 0, never negative."""
    assert reuse.common_prefix([1, 2, 3], []) == 0
    assert reuse.common_prefix([], []) == 0
