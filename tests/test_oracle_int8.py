"""Pins for the INT8 quantizer, the witness bound and RoPE (oracle/int8.py,
oracle/rope.py, oracle/decoder.expected_int8_store).

What pins it:
* the block scale against exact rational arithmetic rounded to the nearest
  float32 by brute force (fractions.Fraction), not numpy;
* each code against a brute-force nearest-integer search with ties to even;
* the absmax element maps to +-127; all-zero blocks give scale 0 and codes 0;
* the bound is sound for every token (Cauchy-Schwarz) and exactly tight for
  adversarial queries aligned band by band with the residual ([WitCert]
  "频带酉性与双层证书": the bound must hold per query, never on averages);
* RoPE band unitarity for interleaved pairs, its failure for half-split
  pairs, and the textbook relative-position property of rotary embeddings;
* exactly quantizable data (zero residual) reduces INT8 attention to the
  plain masked attention;
* the storage format printed on the page (16 bands, 32 B per token-head);
* every field of the expected INT8 ring store (slot positions, key and value
  codes and scales, witness rows) against brute force from exact rationals.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as att
from oracle import decoder, int8, rope


def nearest_f32(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32, ties to even (brute force)."""
    f = np.float32(float(x))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x),
                                     int(np.array(c).view(np.uint32)) & 1))
    return np.float32(best)


def brute_code(x32: np.float32, s: np.float32) -> int:
    quot = Fraction(float(np.float32(x32 / s)))  # the float32 quotient the method fixes
    best = min(range(-127, 128), key=lambda c: (abs(quot - c), c & 1))
    return best


@pytest.mark.parametrize("seed", range(6))
def test_block_scale_and_codes_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((16, 8)) * (10.0 ** rng.uniform(-3, 3))).astype(np.float32)
    if seed == 1:
        x[3, 5] = np.float32(127.5) * np.float32(0.5)  # exercise ties
    s, codes = int8.quantize_block(x)
    a = Fraction(float(np.max(np.abs(x))))
    assert s == nearest_f32(a / 127)
    for idx in np.ndindex(x.shape):
        assert codes[idx] == brute_code(x[idx], s), idx
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert abs(int(codes[i])) == 127
    err = np.abs(x.astype(np.float64) - int8.dequantize(codes, s))
    assert np.all(err <= float(s) / 2 * (1 + 2.0 ** -20))


def test_zero_block():
    s, codes = int8.quantize_block(np.zeros((16, 128), dtype=np.float32))
    assert s == 0 and not codes.any()


def test_round_half_even_ties():
    s = np.float32(1.0)
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 126.5, -126.5, 127.0], dtype=np.float32)
    assert list(int8.block_codes(x, s)) == [0, 2, 2, 0, -2, 126, -126, 127]


def residuals(rng, n, d):
    k = rng.standard_normal((n, d))
    blocks = n // 16
    s, c = int8.quantize_history(k.astype(np.float32), blocks)
    khat = np.concatenate([int8.dequantize(c[i * 16:(i + 1) * 16], s[i]) for i in range(blocks)])
    return k.astype(np.float32).astype(np.float64) - khat


@pytest.mark.parametrize("d", [16, 128])
def test_bound_sound_random_queries(d):
    rng = np.random.default_rng(d)
    r = residuals(rng, 64, d)
    wit = int8.band_norms(r)
    for _ in range(50):
        q = rng.standard_normal(d) * rng.uniform(0.1, 10)
        c = int8.witness_bound(q, wit)
        e = int8.logit_error(q, r)
        assert np.all(c >= e * (1 - 1e-12)), "bound must hold for every token"


@pytest.mark.parametrize("d", [16, 128])
def test_bound_tight_for_aligned_queries(d):
    """q_b = lambda_b * r_b with lambda_b > 0 makes every Cauchy-Schwarz and the
    triangle inequality tight: c_t equals the true error for that token."""
    rng = np.random.default_rng(100 + d)
    r = residuals(rng, 32, d)
    wit = int8.band_norms(r)
    for t in range(32):
        lam = np.repeat(rng.uniform(0.5, 3.0, d // 8), 8)
        q = lam * r[t]
        c = int8.witness_bound(q, wit[t:t + 1])[0]
        e = int8.logit_error(q, r[t:t + 1])[0]
        assert c == pytest.approx(e, rel=1e-12)
        # flipping the sign of one band breaks the triangle-inequality tightness
        q2 = q.copy()
        q2[:8] *= -1
        assert int8.witness_bound(q2, wit[t:t + 1])[0] > int8.logit_error(q2, r[t:t + 1])[0] * (1 + 1e-9)


def test_band_grouping_is_contiguous():
    x = np.zeros(128)
    x[8:16] = 1.0  # band 1 only
    n = int8.band_norms(x)
    assert n[1] == pytest.approx(np.sqrt(8)) and np.count_nonzero(n) == 1


def test_rope_band_unitarity():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 128))
    for pos in [0, 1, 17, 4095, 32767, 131071]:
        y = rope.rope_interleaved(x, pos)
        np.testing.assert_allclose(int8.band_norms(y), int8.band_norms(x), rtol=0, atol=1e-13)
    y = rope.rope_half_split(x, 17)
    assert np.max(np.abs(int8.band_norms(y) - int8.band_norms(x))) > 1e-3


def test_rope_is_a_rotation_by_relative_position():
    """(R_m q) . (R_n k) = (R_{m-n} q) . k, and R_0 is the identity."""
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    np.testing.assert_allclose(rope.rope_interleaved(q, 0), q, atol=0)
    for m, n in [(5, 2), (300, 17), (9000, 8999)]:
        lhs = rope.rope_interleaved(q, m) @ rope.rope_interleaved(k, n)
        rhs = rope.rope_interleaved(q, m - n) @ k
        assert lhs == pytest.approx(rhs, abs=1e-10)


def test_exactly_quantizable_history_reduces_to_plain_attention():
    """Keys/values that are exact multiples of a power-of-two scale with the
    block absmax at +-127 quantize with zero residual: INT8 attention must then
    equal the masked float64 attention, with c = e = 0."""
    rng = np.random.default_rng(9)
    n, d, w = 16 * 5 + 7, 128, 48
    scale = 2.0 ** -5
    k = rng.integers(-127, 128, (n, d)).astype(np.float64)
    v = rng.integers(-127, 128, (n, d)).astype(np.float64)
    k[::16, 0], v[::16, 0] = 127, -127
    k, v = k * scale, v * scale
    q = rng.standard_normal(d)
    res = int8.int8_decode(q, k, v, n, w)
    ref = att.masked_attention(q, np.arange(n), k, v, n - 1, w)
    np.testing.assert_allclose(res["out"], ref, atol=1e-13)
    assert not np.any(res["c"]) and not np.any(res["e"])
    assert list(res["positions"]) == list(range(n - w, n))


def test_int8_decode_staging_and_window():
    rng = np.random.default_rng(10)
    d, w = 128, 64
    for n in [1, 15, 16, 17, 63, 64, 65, 80, 100, 129]:
        k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
        q = rng.standard_normal(d)
        res = int8.int8_decode(q, k, v, n, w)
        ln = min(w, n)
        assert list(res["positions"]) == list(range(n - ln, n))
        exact = res["positions"] >= 16 * (n // 16)
        assert not np.any(res["c"][exact])
        assert np.all(res["c"] >= res["e"] * (1 - 1e-12))
        ref = att.masked_attention(q, np.arange(n), k, v, n - 1, w)
        assert np.max(np.abs(res["out"] - ref)) < 0.05  # quantization error, loose


def test_expected_store_consistent():
    rng = np.random.default_rng(12)
    d, w = 128, 64
    n = 16 * 9 + 5
    k, v = rng.standard_normal((n, d)).astype(np.float32), rng.standard_normal((n, d)).astype(np.float32)
    st = decoder.expected_int8_store(k, v, n, w)
    assert st["staged_positions"] == list(range(144, 149))
    # ring holds the last w/16 complete blocks: positions 80..143
    assert sorted(st["slot_pos"]) == list(range(80, 144))
    for s in range(w):
        p = st["slot_pos"][s]
        assert p % w == s
        blk = p // 16
        sc, codes = int8.quantize_block(k[blk * 16:(blk + 1) * 16])
        assert st["k_scale"][s // 16] == sc
        np.testing.assert_array_equal(st["k_codes"][s], codes[p % 16])


def _brute_block(x32: np.ndarray):
    """Scale and codes of one [16, D] float32 block from exact rationals:
    s = nearest float32 of max|x| / 127; code = nearest integer (ties to even)
    of the nearest float32 of x / s, clamped to +-127; s = 0 gives zeros."""
    a = max(abs(Fraction(float(x))) for x in x32.ravel())
    s = nearest_f32(a / 127)
    if s == 0:
        return s, np.zeros(x32.shape, dtype=np.int64)
    codes = np.zeros(x32.shape, dtype=np.int64)
    for idx in np.ndindex(x32.shape):
        quot = Fraction(float(nearest_f32(Fraction(float(x32[idx])) / Fraction(float(s)))))
        lo = quot.numerator // quot.denominator          # floor
        rest = quot - lo
        c = lo + 1 if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and lo % 2) else lo
        codes[idx] = max(-127, min(127, c))
    return s, codes


@pytest.mark.parametrize("n,w,zero_block", [(16 * 9 + 5, 64, None), (40, 64, 1), (16 * 12, 32, 10),
                                              (16 * 5 + 15, 64, None)])
def test_expected_store_values_and_witness_brute_force(n, w, zero_block):
    """Every stored field of ``expected_int8_store`` against brute force from
    exact rationals, slot by slot: the slot's position (newest committed
    position congruent to the slot), the key and value codes and scales of
    the block that position belongs to, and the witness rows (band norms of
    the exact key residual k - s_K code, compared through their squares,
    exactly).  Covers a wrapped ring, an unfilled one, an all-zero block and
    a history one token short of a block commit."""
    rng = np.random.default_rng(n + w)
    d = 32
    k = (rng.standard_normal((n, d)) * 3).astype(np.float32)
    v = (rng.standard_normal((n, d)) * 0.5).astype(np.float32)
    if zero_block is not None:
        k[zero_block * 16:(zero_block + 1) * 16] = 0
        v[zero_block * 16:(zero_block + 1) * 16] = 0
    st = decoder.expected_int8_store(k, v, n, w)
    nb = n // 16
    blocks = {}
    for blk in range(max(0, nb - w // 16), nb):
        rows = slice(blk * 16, blk * 16 + 16)
        blocks[blk] = (_brute_block(k[rows]), _brute_block(v[rows]))
    for slot in range(w):
        cands = [p for p in range(16 * nb) if p % w == slot]
        want = max(cands) if cands else -1
        assert st["slot_pos"][slot] == want, slot
        if want < 0:
            assert not st["k_codes"][slot].any() and not st["v_codes"][slot].any()
            assert not st["witness"][slot].any()
            continue
        (sk, ck), (sv, cv) = blocks[want // 16]
        r = want % 16
        assert st["k_scale"][slot // 16] == sk and st["v_scale"][slot // 16] == sv, slot
        np.testing.assert_array_equal(st["k_codes"][slot], ck[r])
        np.testing.assert_array_equal(st["v_codes"][slot], cv[r])
        res = [Fraction(float(k[want, c])) - Fraction(float(sk)) * int(ck[r, c]) for c in range(d)]
        for band in range(d // 8):
            exact = sum(x * x for x in res[8 * band:8 * band + 8])
            got = Fraction(float(st["witness"][slot, band])) ** 2
            assert abs(got - exact) <= Fraction(1, 10 ** 14) * exact, (slot, band)
    assert st["staged_positions"] == list(range(16 * nb, n))



@pytest.mark.parametrize("n,w", [(16 * 3 + 5, 40), (16 * 4, 64), (16 * 6 + 15, 200)])
def test_int8_decode_against_brute_force_store(n, w):
    """int8_decode against an independent computation from the brute-force
    block quantizer: keys AND values read as s * code for positions in
    complete blocks and exactly for the staged tail, the masked softmax of
    the window, c_t = (1/sqrt(d)) sum_b ||q_b|| ||r_{t,b}|| per visible token
    (0 when staged), e_t = |q . r_t| / sqrt(d), and cmax = max_t c_t -- which
    for random queries lies strictly above max_t e_t."""
    rng = np.random.default_rng(7 * n + w)
    d = 32
    k = (rng.standard_normal((n, d)) * 2).astype(np.float32).astype(np.float64)
    v = (rng.standard_normal((n, d)) * 0.7).astype(np.float32).astype(np.float64)
    q = rng.standard_normal(d)
    res = int8.int8_decode(q, k, v, n, w)
    nb = n // 16
    k_hat, v_hat = k.copy(), v.copy()
    for blk in range(nb):
        rows = slice(16 * blk, 16 * blk + 16)
        (sk, ck), (sv, cv) = _brute_block(k[rows].astype(np.float32)), _brute_block(v[rows].astype(np.float32))
        k_hat[rows] = float(sk) * ck
        v_hat[rows] = float(sv) * cv
    ln = min(w, n)
    vis = np.arange(n - ln, n)
    sc = k_hat[vis] @ q / np.sqrt(d)
    p = np.exp(sc - sc.max())
    out = (p / p.sum()) @ v_hat[vis]
    np.testing.assert_allclose(res["out"], out, rtol=0, atol=1e-12)
    r = k[vis] - k_hat[vis]
    qn = np.sqrt((q.reshape(-1, 8) ** 2).sum(axis=1))
    c = np.array([sum(qn[b] * np.sqrt((r[i, 8 * b:8 * b + 8] ** 2).sum()) for b in range(d // 8))
                  for i in range(ln)]) / np.sqrt(d)
    e = np.abs(r @ q) / np.sqrt(d)
    np.testing.assert_allclose(res["c"], c, rtol=1e-12, atol=0)
    np.testing.assert_allclose(res["e"], e, rtol=1e-12, atol=1e-300)
    assert not np.any(res["c"][vis >= 16 * nb]), "staged tokens are exact"
    assert res["cmax"] == pytest.approx(c.max(), rel=1e-12)
    assert res["cmax"] > e.max() * (1 + 1e-6)


def test_int8_decode_single_visible_token_is_its_dequantized_value():
    """A window of one slot whose token sits in a complete block: the output
    is that token's value row s_V * code exactly (softmax of one logit is 1)."""
    rng = np.random.default_rng(31)
    d = 32
    k = rng.standard_normal((16, d)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((16, d)).astype(np.float32).astype(np.float64)
    res = int8.int8_decode(rng.standard_normal(d), k, v, 16, 1)
    sv, cv = _brute_block(v.astype(np.float32))
    np.testing.assert_array_equal(res["out"], float(sv) * cv[15])
    assert not np.array_equal(res["out"], v[15]), "the value row is read quantized"


def test_storage_format(golden):
    g = golden("witcert_witness_format.json")
    d = g["head_dim"]
    nb = d // int8.BAND
    assert nb == g["bands"]
    assert nb * 2 == g["witness_bytes_per_token_head"]  # fp16 per band
    per_token_head = 2 * d * 1 + nb * 2 + 2 * 4 / int8.BLOCK  # codes K+V, witness, scales
    assert per_token_head == 288.5


def test_codes_use_correctly_rounded_division_near_ties():
    """Near rounding ties the float32 quotient x/s (correctly rounded, computed
    here from exact rationals) decides the code; a reciprocal multiply would
    differ on some of these inputs."""
    rng = np.random.default_rng(77)
    checked = 0
    for _ in range(400):
        s = np.float32(rng.uniform(0.01, 0.05))
        k = int(rng.integers(-126, 126))
        x0 = np.float32((k + 0.5) * float(s))
        for x in (np.nextafter(x0, np.float32(-1e9)), x0, np.nextafter(x0, np.float32(1e9))):
            quot = nearest_f32(Fraction(float(x)) / Fraction(float(s)))
            expect = min(range(-127, 128), key=lambda c: (abs(Fraction(float(quot)) - c), c & 1))
            assert int(int8.block_codes(np.array([x], dtype=np.float32), s)[0]) == expect
            checked += 1
    assert checked == 1200


def test_rope_angle_from_definition():
    """theta_i = base^(-2i/D): with D = 128 and base 10000, pair i = 32 turns by
    exactly 10000^(-1/2) = 0.01 rad per position; pair 0 by 1 rad."""
    e = np.zeros(128)
    e[64] = 1.0
    y = rope.rope_interleaved(e, 1)
    assert y[64] == pytest.approx(np.cos(0.01), abs=1e-15) and y[65] == pytest.approx(np.sin(0.01), abs=1e-15)
    e0 = np.zeros(128)
    e0[0] = 1.0
    y0 = rope.rope_interleaved(e0, 3)
    assert y0[0] == pytest.approx(np.cos(3.0), abs=1e-15) and y0[1] == pytest.approx(np.sin(3.0), abs=1e-15)


def test_rope_half_split_is_the_interleaved_rotation_on_reordered_dims():
    """The half-split form rotates the pairs (i, i + D/2) by the same angles
    that the interleaved form applies to (2i, 2i + 1): reorder the dims so
    those pairs become adjacent and the two agree exactly; both preserve the
    norm of the whole vector."""
    rng = np.random.default_rng(21)
    d = 32
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 100, 32767])
    h = d // 2
    perm = np.empty(d, dtype=np.int64)
    perm[0::2], perm[1::2] = np.arange(h), np.arange(h) + h      # y[2i] = x[i], y[2i+1] = x[i + D/2]
    got = rope.rope_half_split(x, pos)
    want = np.empty_like(x)
    want[:, perm] = rope.rope_interleaved(x[:, perm], pos)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
