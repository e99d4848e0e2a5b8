"""Pins for the reference attention and the full-history decoder.

What pins it:
* an independent library routine: torch's scaled_dot_product_attention on
  the CPU in float64 with an explicit boolean mask (a transposed operand, a
  wrong scale or sign, or a dropped mask term would differ);
* closed forms of softmax attention (one visible token, zero query,
  identical keys, one dominant key);
* the [KV-Loop] three-step example (tests/golden/kv_loop_three_steps.json);
* the theorem of [Lean-SWA] §4.2 (windowed cache attention = masked
  full-history attention) on the tiny W=4 workload and a brute-force sweep,
  to the frozen 1e-12 threshold of [Prefix-Reuse] "27 例".
"""

import numpy as np
import pytest
import torch

import workloads
from workloads import gen
from oracle import attention as att
from oracle import bits, decoder, listmodel
from oracle import int8 as oint8


def sdpa_reference(q, pos, k, v, t, w):
    """torch SDPA (float64, CPU) with the window+causal mask as a bool mask."""
    mask = torch.from_numpy(((pos >= t - w + 1) & (pos <= t))[None, :])
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[None, None, :]), torch.from_numpy(k[None]), torch.from_numpy(v[None]),
        attn_mask=mask[None])
    return out[0, 0].numpy()


@pytest.mark.parametrize("n,w,d", [(1, 4, 16), (7, 4, 16), (33, 8, 32), (200, 64, 128), (50, 100, 8)])
def test_masked_attention_matches_library(n, w, d):
    rng = np.random.default_rng(n * 1000 + w)
    q, k, v = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    pos = np.arange(n)
    for t in sorted({0, n // 2, n - 1}):
        got = att.masked_attention(q, pos, k, v, t, w)
        ref = sdpa_reference(q, pos, k, v, t, w)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(5)
    d = 16
    k, v = rng.standard_normal((9, d)), rng.standard_normal((9, d))
    # one visible token: the output is exactly its value row
    np.testing.assert_array_equal(att.plain_attention(rng.standard_normal(d), k[:1], v[:1]), v[0])
    # zero query: uniform weights, the mean of V
    np.testing.assert_allclose(att.plain_attention(np.zeros(d), k, v), v.mean(axis=0), atol=1e-15)
    # identical keys: uniform weights for any query
    np.testing.assert_allclose(att.plain_attention(rng.standard_normal(d), np.tile(k[:1], (9, 1)), v),
                               v.mean(axis=0), atol=1e-14)
    # one key scaled x1000 along the query: the output is that key's value row
    q = rng.standard_normal(d)
    k2 = k.copy()
    k2[4] = 1000.0 * q / np.linalg.norm(q)
    np.testing.assert_allclose(att.plain_attention(q, k2, v), v[4], atol=1e-12)
    # empty visible set (pages silent): zeros
    assert not att.masked_attention(q, np.arange(3), k[:3], v[:3], -1, 4).any()


def test_three_step_example(golden):
    g = golden("kv_loop_three_steps.json")
    rng = np.random.default_rng(0)
    H, D, B = g["num_heads"], g["head_dim"], g["batch"]
    hist = [decoder.SequenceHistory(H, D) for _ in range(B)]
    for _ in range(g["steps"]):
        outs = []
        for b in range(B):
            hist[b].append(rng.standard_normal((H, 1, D)), rng.standard_normal((H, 1, D)))
            outs.append(hist[b].attend(rng.standard_normal((H, D)), g["max_seq_len"]))
        out = np.stack(outs)[:, :, None, :]
        assert list(out.shape) == g["expected_out_shape"]
    assert all(h.next_position == g["expected_current_len"] for h in hist)


def tiny_inputs():
    wl = workloads.TINY
    n = wl.steps
    k = bits.to_f64(gen.to_bits(gen.tokens(wl, "k", n)))
    v = bits.to_f64(gen.to_bits(gen.tokens(wl, "v", n)))
    qs = [bits.to_f64(gen.to_bits(gen.query(wl, t))) for t in range(n)]
    return wl, k, v, qs


def test_tiny_workload_window_equals_full_history():
    """W=4, 12 steps from empty: unfilled (t=0..2), exactly full (t=3), first
    overwrite (t=4), then wraps; every step the cache-window attention equals
    the masked full-history attention to 1e-12 and the window positions
    follow pos_i = t - len + 1 + i."""
    wl, k, v, qs = tiny_inputs()
    hist = decoder.SequenceHistory(wl.H, wl.D)
    for t in range(wl.steps):
        hist.append(k[0, :, t:t + 1], v[0, :, t:t + 1])
        full = hist.attend(qs[t][0], wl.W)
        win = hist.attend_window(qs[t][0], wl.W)
        assert np.max(np.abs(full - win)) <= 1e-12
        ring = decoder.expected_ring(np.arange(t + 1), wl.W)
        assert listmodel.ring_to_list(wl.W, list(ring), t + 1) == listmodel.window_positions(wl.W, t)


@pytest.mark.parametrize("w", range(1, 7))
def test_brute_force_theorem_with_chunked_appends(w):
    """Appends in chunks of T = 1..2W+1 tokens up to 4W tokens: after each
    chunk, windowed = full masked attention and the expected ring slots hold
    exactly the last-window positions."""
    rng = np.random.default_rng(w)
    H, D = 1, 8
    for T in range(1, 2 * w + 2):
        hist = decoder.SequenceHistory(H, D)
        while hist.next_position < 4 * w:
            hist.append(rng.standard_normal((H, T, D)), rng.standard_normal((H, T, D)))
            q = rng.standard_normal((H, D))
            assert np.max(np.abs(hist.attend(q, w) - hist.attend_window(q, w))) <= 1e-12
            n = hist.next_position
            ring = decoder.expected_ring(np.arange(n), w)
            assert sorted(int(p) for p in ring if p >= 0) == listmodel.window_positions(w, n - 1)


def test_stale_next_position_is_a_large_error():
    """Negative control of [Prefix-Reuse] "哪些東西必須一起裁剪": keeping the
    prefix rows but a stale next_position shifts every position, so the window
    covers other rows and the error is far above rounding."""
    rng = np.random.default_rng(11)
    d, w = 16, 4
    k, v = rng.standard_normal((12, d)), rng.standard_normal((12, d))
    q = rng.standard_normal(d)
    good = att.masked_attention(q, np.arange(12), k, v, 11, w)
    stale = att.masked_attention(q, np.arange(12) + 4, k, v, 11, w)
    assert np.max(np.abs(good - stale)) > 1e-2


def test_empty_visible_set_gives_zeros():
    """R7: an empty cache (or an empty visible set) answers with the zero
    vector, through every oracle entry point that can see one."""
    d = 16
    q = np.ones(d)
    empty = np.zeros((0, d))
    assert not np.any(att.plain_attention(q, empty, empty))
    assert att.plain_attention(q, empty, empty).shape == (d,)
    assert not np.any(att.masked_attention(q, np.arange(0), empty, empty, -1, 4))
    hist = decoder.SequenceHistory(2, d)
    assert not np.any(hist.attend(np.ones((2, d)), 4))
    assert not np.any(hist.attend_window(np.ones((2, d)), 4))
    empty128 = np.zeros((0, 128))
    assert not np.any(oint8.int8_decode(np.ones(128), empty128, empty128, 0, 16)["out"])


def test_masking_is_exact_at_large_logit_magnitudes():
    """Invisible rows get exactly zero weight however large the visible
    logits are in magnitude: with every visible logit near -1e4 (or +1e4) and
    invisible rows present, the masked attention equals plain attention over
    the visible rows alone."""
    rng = np.random.default_rng(12)
    d, n, w = 16, 12, 4
    for sign in (-1.0, 1.0):
        q = np.ones(d) * 100.0
        k = rng.standard_normal((n, d)) * 0.01 + sign * 25.0   # q.k/sqrt(d) ~ sign * 1e4
        v = rng.standard_normal((n, d))
        t = n - 1
        got = att.masked_attention(q, np.arange(n), k, v, t, w)
        want = att.plain_attention(q, k[t - w + 1:], v[t - w + 1:])
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
