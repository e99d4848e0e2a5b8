"""Pins for the Tier B oracle (oracle/philox.py, oracle/dither.py).

What pins it:
* Philox-4x32-10 against the known-answer vectors published with the
  generator (Salmon et al., SC 2011; Random123 known-answer tests): zero
  counter and key, all-ones, and the digits-of-pi vector;
* the same round function at 64-bit width against NumPy's own Philox-4x64-10
  bit generator, an independent implementation (NumPy advances its
  counter by one before each block);
* the vectorized form against the scalar form on random counters and keys;
* the dither byte order through the zero-vector known answer, and the
  placement of the five-tuple in counter and key through the pi vector;
* the quantizer: ties go to the even code (brute force); keys and values
  share the dither; with zero dither it is Tier A's quantizer; over all 256
  dither values of one element the residual is a contiguous 256-point grid
  of spacing 1/256 whose mean is within BETA of 0 and whose variance is
  exactly (1 - 2^-16)/12 (brute force with exact rationals);
* the sub-Gaussian constant: the log moment generating function of that
  grid law is at most lambda^2/24 (the 1/12 variance proxy), and the ratio
  tends to its variance at small lambda;
* the certificate: its scale against the Monte Carlo standard deviation of
  the logit error over independent dither streams, its coverage (no
  violations at the stated budget) and its tightness (the largest
  error reaches most of the bound), all through int8_dither_decode;
* the bias term: with a budget that makes the concentration term vanish,
  the certificate still covers the exact mean logit error over the dither
  (all 256 values per channel enumerated) where that mean is largest;
* decode special cases: no complete block -> exact attention and a zero
  certificate; empty history -> zeros; a one-hot query returns its value
  row within half a step; a one-slot window returns the stored value row
  s (code - u) exactly.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as att
from oracle import dither, int8, philox

# Known answers of Philox-4x32-10 (counter, key, output), as published with
# the generator's reference implementation.
KAT_4X32 = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT_4X32)
def test_philox4x32_known_answers(ctr, key, want):
    assert philox.philox(ctr, key, 32) == want
    got = philox.philox4x32(np.array(ctr, dtype=np.uint64), np.array(key, dtype=np.uint64))
    assert tuple(int(x) for x in got) == want


@pytest.mark.parametrize("seed", range(4))
def test_philox4x64_matches_numpy(seed):
    rng = np.random.default_rng(seed)
    ctr = [int(rng.integers(0, 1 << 62)), int(rng.integers(0, 1 << 63)), int(rng.integers(0, 1 << 63)),
           int(rng.integers(0, 1 << 63))]
    key = [int(rng.integers(0, 1 << 63)), int(rng.integers(0, 1 << 63))]
    bg = np.random.Philox(counter=ctr, key=key)
    raw = [int(x) for x in bg.random_raw(8)]
    want0 = philox.philox([ctr[0] + 1] + ctr[1:], key, 64)
    want1 = philox.philox([ctr[0] + 2] + ctr[1:], key, 64)
    assert tuple(raw[:4]) == want0
    assert tuple(raw[4:]) == want1


def test_philox_vectorized_matches_scalar():
    rng = np.random.default_rng(7)
    ctr = rng.integers(0, 1 << 32, size=(50, 4), dtype=np.uint64)
    key = rng.integers(0, 1 << 32, size=(50, 2), dtype=np.uint64)
    got = philox.philox4x32(ctr, key)
    for i in range(50):
        assert tuple(int(x) for x in got[i]) == philox.philox(ctr[i], key[i], 32)
    # broadcasting one key over many counters
    got_b = philox.philox4x32(ctr, key[0])
    assert tuple(int(x) for x in got_b[3]) == philox.philox(ctr[3], key[0], 32)


def test_dither_byte_order_from_known_answer():
    # request 0, layer 0, head 0, position 0, channels 0..15 -> counter 0, key 0
    m = dither.dither_bytes(0, 0, 0, [0], 16)[0]
    want = []
    for w in KAT_4X32[0][2]:
        want += [(w >> (8 * i)) & 0xFF for i in range(4)]
    assert list(m) == want
    u = dither.dither_values(m)
    assert np.all(np.abs(u) < 0.5) and np.all(((0.5 - u) * 256 - 0.5) == m)


def test_tuple_fields_from_known_answer():
    # The digits-of-pi vector gives every counter and key word a distinct
    # value: request 0x299F31D0_A4093822, layer 0x03707344, head 0x13198A2E,
    # position 0x243F6A88, channel group 0x85A308D3.
    ctr = dither.philox_counter(0x03707344, 0x13198A2E, 0x243F6A88, 0x85A308D3)
    key = dither.philox_key(0x299F31D0A4093822)
    got = philox.philox4x32(ctr, key)
    assert tuple(int(x) for x in got) == KAT_4X32[2][2]
    # dither_bytes uses that layout for every (token, group)
    m = dither.dither_bytes(0x299F31D0A4093822, 7, 9, [3, 1000], 48)
    for i, pos in enumerate((3, 1000)):
        for g in range(3):
            words = philox.philox4x32(dither.philox_counter(7, 9, pos, g), key)
            assert np.array_equal(m[i, 16 * g:16 * g + 16], dither.group_bytes(words)[0])


def test_dither_stream_is_uniform_and_keyed():
    m = dither.dither_bytes(12345, 3, 5, np.arange(4096), 128).astype(np.int64)
    counts = np.bincount(m.ravel(), minlength=256)
    expect = m.size / 256
    chi2 = float(np.sum((counts - expect) ** 2 / expect))
    assert chi2 < 400  # 255 degrees of freedom; p ~ 1e-8 above this
    # neighbouring channels and tokens are uncorrelated
    u = dither.dither_values(m)
    assert abs(np.corrcoef(u[:, :-1].ravel(), u[:, 1:].ravel())[0, 1]) < 0.01
    assert abs(np.corrcoef(u[:-1].ravel(), u[1:].ravel())[0, 1]) < 0.01
    # every tuple member moves the stream
    base = dither.dither_bytes(12345, 3, 5, [77], 32)
    for other in (dither.dither_bytes(12346, 3, 5, [77], 32), dither.dither_bytes(12345, 4, 5, [77], 32),
                  dither.dither_bytes(12345, 3, 6, [77], 32), dither.dither_bytes(12345, 3, 5, [78], 32),
                  dither.dither_bytes(12345 + (1 << 32), 3, 5, [77], 32)):
        assert np.mean(base == other) < 0.1
    # the stream of a token does not depend on which other tokens are asked for
    assert np.array_equal(dither.dither_bytes(9, 1, 2, [5, 40, 41], 64)[1],
                          dither.dither_bytes(9, 1, 2, [40], 64)[0])
    # channel groups are distinct counters
    wide = dither.dither_bytes(9, 1, 2, [40], 64)[0]
    assert np.mean(wide[:16] == wide[16:32]) < 0.2


@pytest.mark.parametrize("seed", range(4))
def test_zero_dither_is_tier_a(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((16, 32)) * 3).astype(np.float32)
    s, c = dither.quantize_block(x, np.zeros_like(x, dtype=np.float64))
    s_a, c_a = int8.quantize_block(x)
    assert s == s_a and np.array_equal(c, c_a)


def test_clamp_never_acts_and_round_trip():
    rng = np.random.default_rng(3)
    for trial in range(20):
        x = (rng.standard_normal((16, 64)) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32)
        x[0, 0] = np.max(np.abs(x)) * (1 if trial % 2 else -1)  # the absmax with either sign
        m = rng.integers(0, 256, size=x.shape)
        m[0, 0] = 255 if trial % 2 else 0                      # extreme dither on the absmax
        u = dither.dither_values(m)
        s = int8.block_scale(x)
        t = x / np.float32(s) + u.astype(np.float32)
        assert np.max(np.abs(np.rint(t))) <= 127                # before the clamp
        c = dither.block_codes(x, s, u)
        err = np.abs(dither.dequantize(c, s, u) - x.astype(np.float64))
        assert np.all(err <= float(s) * (0.5 + 2.0 ** -16))


def test_ties_round_to_even():
    # s = 1 exactly (absmax 127); y + u lands on k + 1/2 for the chosen
    # elements: code = the even neighbour (brute force over candidates).
    x = np.zeros(16, dtype=np.float32)
    x[0] = 127
    u = np.zeros(16)
    m = 64                                                     # u = 1/4 - 1/512
    for j, y in enumerate([2.25 + 1 / 512, 3.25 + 1 / 512, -2.75 + 1 / 512, -5.75 + 1 / 512], start=1):
        x[j] = y
        u[j] = dither.dither_values(m)
    s = int8.block_scale(x)
    assert s == 1
    c = dither.block_codes(x, s, u)
    for j in range(1, 5):
        t = Fraction(float(x[j])) + Fraction(float(u[j]))
        assert t.denominator == 2                              # an exact tie
        cands = [int(t - Fraction(1, 2)), int(t + Fraction(1, 2))]
        assert int(c[j]) == [cc for cc in cands if cc % 2 == 0][0]


def test_keys_and_values_share_the_dither():
    rng = np.random.default_rng(4)
    n, d = 48, 128
    kv = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    r = dither.int8_dither_decode(rng.standard_normal(d), kv, kv.copy(), n, n, request=3, layer=1, head=2,
                                  delta=0.1)
    assert np.array_equal(r["k_codes"], r["v_codes"]) and np.array_equal(r["k_scales"], r["v_scales"])


def test_one_hot_query_returns_the_dequantized_value():
    # Key j is the only one aligned with q (logit ~ 90 above the rest), so the
    # output is value row j as stored: within s_V (1/2 + BETA) of the input.
    rng = np.random.default_rng(6)
    n, d = 40, 128
    q = np.zeros(d)
    q[:8] = 1.0
    for j in (0, 17, 31):
        k = np.zeros((n, d))
        k[j, :8] = 1024.0
        v = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
        r = dither.int8_dither_decode(q, k, v, n, n, request=11, layer=0, head=0, delta=0.1)
        sv = float(r["v_scales"][j // 16])
        assert np.max(np.abs(r["out"] - v[j])) <= sv * (0.5 + dither.BETA) + 1e-12


def test_zero_block_codes():
    x = np.zeros((16, 32), dtype=np.float32)
    s, c = dither.quantize_block(x, dither.dither_values(np.full(x.shape, 200)))
    assert s == 0 and not c.any()
    assert not dither.dequantize(c, s, dither.dither_values(np.full(x.shape, 200))).any()


@pytest.mark.parametrize("seed", range(8))
def test_residual_is_a_contiguous_grid_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    x = (rng.standard_normal(16) * 5).astype(np.float32)
    s = int8.block_scale(x)
    z = Fraction(float(x[seed])) / Fraction(float(s))           # exact x / s
    m = np.arange(256)
    u = dither.dither_values(m)
    codes = dither.block_codes(np.full(256, x[seed], dtype=np.float32), s, u)
    eps = sorted(Fraction(int(c)) - Fraction(float(uu)) - z for c, uu in zip(codes, u))
    h = Fraction(1, 256)
    assert all(b - a == h for a, b in zip(eps, eps[1:]))      # 256 consecutive grid points
    mean = sum(eps) / 256
    assert abs(mean) <= Fraction(dither.BETA)
    var = sum((e - mean) ** 2 for e in eps) / 256
    assert var == (1 - h * h) / 12


def test_grid_law_is_strictly_sub_gaussian():
    pts = (np.arange(256) - 127.5) / 256                          # centred grid law
    var = float(np.mean(pts ** 2))
    assert var == pytest.approx((1 - 2.0 ** -16) / 12, rel=1e-15)
    for lam in np.concatenate([np.linspace(0.01, 5, 50), np.linspace(5, 400, 80)]):
        a = lam * pts
        log_mgf = float(np.max(a) + np.log(np.mean(np.exp(a - np.max(a)))))
        assert log_mgf <= lam * lam / 24 * (1 + 1e-12)
    lam = 1e-3
    log_mgf = float(np.log(np.mean(np.exp(lam * pts))))
    assert log_mgf / (lam * lam / 2) == pytest.approx(var, rel=1e-5)


def test_certificate_scale_matches_monte_carlo_spread():
    # One key row, many independent dither streams (requests): the logit
    # error's spread fixes the bound's Gaussian part.  8000 draws estimate
    # the spread to about 0.8% (relative standard error 1/sqrt(2N)), so the
    # 2.5% tolerance holds the bound's scale factor, union-bound term
    # included, to within about 3 standard errors; ln(n_q/delta) in place of
    # ln(2 n_q/delta) would move it by 4.4%.
    rng = np.random.default_rng(11)
    d, n, delta = 128, 16, 0.01
    k = rng.standard_normal((n, d))
    k = np.asarray(k, dtype=np.float32).astype(np.float64)
    v = np.zeros((n, d))
    q = rng.standard_normal(d)
    errs = []
    for req in range(8000):
        r = dither.int8_dither_decode(q, k, v, n, n, request=req, layer=0, head=0, delta=delta)
        errs.append((r["k_codes"][0].astype(np.float64) - dither.dither_values(r["m"][0])) * float(r["k_scales"][0])
                    - k[0])
    e = np.array([np.dot(er, q) / np.sqrt(d) for er in errs])
    sigma = float(np.std(e))
    s0 = float(dither.int8.block_scale(k))
    bias = s0 / np.sqrt(d) * np.sum(np.abs(q)) * dither.BETA
    c = float(dither.token_bound(q, np.array([s0]), 16, delta)[0])
    gauss = (c - bias) / np.sqrt(2 * np.log(2 * 16 / delta))
    assert gauss / sigma == pytest.approx(1.0, abs=0.025)
    assert abs(float(np.mean(e))) <= bias + 4 * sigma / np.sqrt(len(e))


def test_certificate_coverage_and_tightness():
    rng = np.random.default_rng(5)
    d, w, delta = 128, 256, 0.05
    ratios = []
    violations = 0
    for trial in range(60):
        n = int(rng.integers(200, 300))
        k = (rng.standard_normal((n, d)) * rng.uniform(0.1, 3)).astype(np.float32).astype(np.float64)
        v = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
        q = (rng.standard_normal(d) * rng.uniform(0.2, 2)).astype(np.float32).astype(np.float64)
        r = dither.int8_dither_decode(q, k, v, n, w, request=trial, layer=2, head=1, delta=delta)
        qd = r["c"] > 0
        ratio = r["e"][qd] / r["c"][qd]
        violations += int(np.any(ratio > 1))
        ratios.append(float(np.max(ratio)))
        assert r["cert"] == pytest.approx(float(np.max(r["c"])))
        assert np.all(r["e"][~qd] == 0)  # exact staging tokens
    assert violations == 0
    assert 0.55 < float(np.median(ratios)) < 1.0


def test_decode_without_complete_block_is_exact():
    rng = np.random.default_rng(2)
    d = 128
    for n in (1, 7, 15):
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d))
        q = rng.standard_normal(d)
        r = dither.int8_dither_decode(q, k, v, n, 64, request=1, layer=0, head=0, delta=0.1)
        want = att.plain_attention(q, k, v)
        assert np.allclose(r["out"], want, rtol=0, atol=1e-12)
        assert r["cert"] == 0 and r["n_q"] == 0
    r = dither.int8_dither_decode(np.ones(d), np.zeros((0, d)), np.zeros((0, d)), 0, 64, 1, 0, 0, 0.1)
    assert not r["out"].any() and r["cert"] == 0


def test_decode_within_tv_of_exact_attention():
    # out - exact = sum (p^ - p) v^ + sum p (v^ - v): the first term is at most
    # 2 tanh(E/2) max|v^| with E the largest logit error, the second at most
    # the largest dequantization error s_V (1/2 + BETA).
    rng = np.random.default_rng(9)
    d, w = 128, 96
    for trial in range(10):
        n = int(rng.integers(100, 200))
        k = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
        v = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
        q = (rng.standard_normal(d) * 0.7).astype(np.float32).astype(np.float64)
        r = dither.int8_dither_decode(q, k, v, n, w, request=50 + trial, layer=0, head=3, delta=1e-3)
        vis = r["positions"]
        exact = att.plain_attention(q, k[vis], v[vis])
        vmax = float(np.max(np.abs(v[vis]))) + float(np.max(r["v_scales"]))
        bound = 2 * np.tanh(r["cert"] / 2) * vmax + float(np.max(r["v_scales"])) * (0.5 + dither.BETA)
        assert np.max(np.abs(r["out"] - exact)) <= bound


def test_position_offset_is_the_same_history_further_on():
    # Rows at positions P0 + j: with n >= W only the last W rows are visible,
    # so this equals the history padded with P0 leading rows.
    rng = np.random.default_rng(12)
    d, w, p0, n = 128, 64, 48, 100
    k = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    q = rng.standard_normal(d)
    a = dither.int8_dither_decode(q, k, v, n, w, request=5, layer=2, head=1, delta=0.1, position0=p0)
    pad = np.zeros((p0, d))
    b = dither.int8_dither_decode(q, np.concatenate([pad, k]), np.concatenate([pad, v]), p0 + n, w, request=5, layer=2,
                                  head=1, delta=0.1)
    assert np.array_equal(a["out"], b["out"]) and a["cert"] == b["cert"]
    assert np.array_equal(a["k_codes"][-w:], b["k_codes"][-w:])


def test_one_slot_window_returns_the_stored_value_row_exactly():
    """A one-slot window over a complete block: softmax of one logit is 1, so
    the output is the stored value row s_V (code - u), with the scale and the
    codes re-derived here from their definition (absmax / 127 rounded to
    float32 from exact rationals; the nearest integer, ties to even, of the
    float32 sum f32(x / s) + u)."""
    rng = np.random.default_rng(41)
    d = 32
    k = rng.standard_normal((16, d)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((16, d)).astype(np.float32).astype(np.float64)
    r = dither.int8_dither_decode(rng.standard_normal(d), k, v, 16, 1, request=5, layer=2, head=1, delta=0.1)
    u = dither.dither(5, 2, 1, [15], d)[0]
    v32 = v.astype(np.float32)
    a = max(abs(Fraction(float(x))) for x in v32.ravel()) / 127
    s = np.float32(float(a))
    s = min((s, np.nextafter(s, np.float32(np.inf)), np.nextafter(s, np.float32(-np.inf))),
            key=lambda c: (abs(Fraction(float(c)) - a), int(np.array(c).view(np.uint32)) & 1))
    want = np.empty(d)
    for c in range(d):
        t = Fraction(float(np.float32(np.float32(v32[15, c] / s) + np.float32(u[c]))))
        lo = t.numerator // t.denominator
        rest = t - lo
        code = lo + 1 if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and lo % 2) else lo
        want[c] = float(Fraction(float(s)) * (code - Fraction(float(u[c]))))
    np.testing.assert_array_equal(r["out"], want)
    assert not np.array_equal(r["out"], v[15]), "the value row is read quantized"


def test_certificate_bias_term_covers_the_exact_mean_error():
    """With delta = 2 n_q the concentration term vanishes (ln 1 = 0) and the
    certificate is its bias term (s / sqrt(d)) ||q||_1 beta.  It must cover
    the exact mean of the logit error over the dither, (s / sqrt(d))
    sum_c q_c mu_c, where mu_c is the mean residual of channel c over all 256
    dither values (channels are independent, so means add).  Every channel
    is put at the fractional offset of x / s whose mean residual is largest,
    and q follows its sign, so the mean error is d times one channel's."""
    d = 32
    s0 = 2.0 ** -4                                   # absmax 127 * s0 gives the scale s0 exactly
    u = dither.dither_values(np.arange(256))
    best, best_mu = None, 0.0
    for i in range(512):
        x = np.float32((10 + i / 512) * s0)
        z = float(x) / s0                            # exact: dyadic
        codes = dither.block_codes(np.full(256, x, dtype=np.float32), np.float32(s0), u)
        mu = float(np.mean(codes.astype(np.float64) - u - z))
        if abs(mu) > abs(best_mu):
            best, best_mu = x, mu
    assert abs(best_mu) > dither.BETA / np.sqrt(d) * 2, "the bias term matters at this offset"
    assert abs(best_mu) <= dither.BETA
    block = np.zeros((16, d), dtype=np.float32)
    block[0, 0] = np.float32(127 * s0)
    block[15, :] = best
    assert dither.block_codes(block, int8.block_scale(block), np.zeros((16, d))).any()
    assert int8.block_scale(block) == np.float32(s0)
    q = np.full(d, np.sign(best_mu))
    mean_err = abs(s0 / np.sqrt(d) * float(np.sum(q * best_mu)))
    bound = float(dither.token_bound(q, np.array([s0]), 1, 2.0)[0])
    assert bound >= mean_err
    assert bound == pytest.approx(s0 / np.sqrt(d) * d * dither.BETA, rel=1e-12)


def _nearest_int_even(t: Fraction) -> int:
    lo = t.numerator // t.denominator
    rest = t - lo
    return lo + 1 if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and lo % 2) else lo


def test_decode_errors_and_bounds_against_a_brute_force_store():
    """Through int8_dither_decode, at a budget delta = 2 n_q that zeroes the
    concentration term: every visible token's true logit error
    |q . (k - k_hat)| / sqrt(d) and bound (s_K / sqrt(d)) ||q||_1 beta (0 for
    the exact staged tokens), n_q and the certificate (their maximum), with
    k_hat = s (code - u) re-derived here from the definitions of the scale
    and the codes (exact rationals; float32 steps as the method fixes them)
    and u from the Philox stream."""
    rng = np.random.default_rng(55)
    n, w, d = 16 * 3 + 5, 40, 32
    req, layer, head = 77, 3, 1
    k = (rng.standard_normal((n, d)) * 2).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((n, d)).astype(np.float32).astype(np.float64)
    q = rng.standard_normal(d)
    vis = np.arange(n - w, n)
    quant = vis < 16 * (n // 16)
    n_q = int(quant.sum())
    res = dither.int8_dither_decode(q, k, v, n, w, req, layer, head, delta=2.0 * n_q)
    assert res["n_q"] == n_q
    u = dither.dither(req, layer, head, np.arange(16 * (n // 16)), d)
    k_hat = k.copy()
    s_tok = np.zeros(n)
    for blk in range(n // 16):
        rows = slice(16 * blk, 16 * blk + 16)
        x32 = k[rows].astype(np.float32)
        a = max(abs(Fraction(float(x))) for x in x32.ravel()) / 127
        s = np.float32(float(a))
        s = min((s, np.nextafter(s, np.float32(np.inf)), np.nextafter(s, np.float32(-np.inf))),
                key=lambda c: (abs(Fraction(float(c)) - a), int(np.array(c).view(np.uint32)) & 1))
        for i in range(16):
            for c in range(d):
                t = Fraction(float(np.float32(np.float32(x32[i, c] / s) + np.float32(u[16 * blk + i, c]))))
                code = max(-127, min(127, _nearest_int_even(t)))
                k_hat[16 * blk + i, c] = float(Fraction(float(s)) * (code - Fraction(float(u[16 * blk + i, c]))))
        s_tok[rows] = float(s)
    e = np.abs((k[vis] - k_hat[vis]) @ q) / np.sqrt(d)
    c = np.where(quant, s_tok[vis] / np.sqrt(d) * np.sum(np.abs(q)) * dither.BETA, 0.0)
    np.testing.assert_allclose(res["e"], e, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(res["c"], c, rtol=1e-12, atol=0)
    assert res["cert"] == pytest.approx(c.max(), rel=1e-12)
