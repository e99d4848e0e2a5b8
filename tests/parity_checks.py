"""Comparisons of the HIP results with the oracle, on host arrays only.

These functions take NumPy arrays (the GPU's results already copied to the
host, and the float64 inputs) and import neither torch nor the HIP library,
so the host process pool in ``tests/oracle_pool.py`` can run them too.
"""

from __future__ import annotations

import numpy as np

from oracle import bits, decoder, dither as odither, int8 as oint8

TOL = 2e-3  # max abs error of outputs vs the float64 oracle on the same inputs


def oracle_out(k64: np.ndarray, v64: np.ndarray, q64: np.ndarray, n: int, W: int) -> np.ndarray:
    """Masked full-history attention of the query at step n-1 for every head:
    k64, v64 [H, >=n, D]; q64 [H, D]."""
    hist = decoder.SequenceHistory(k64.shape[0], k64.shape[2])
    hist.append(k64[:, :n], v64[:, :n])
    return hist.attend(q64, W)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, tol: float = TOL):
    err = float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) if ref.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol}"
    return err


def check_int8_store_arrays(kc, vc, ks, vs, wit, pos, ksg, vsg, k64: np.ndarray, v64: np.ndarray, n: int, W: int,
                            what: str = ""):
    """INT8 store of one (sequence, head) in ring order: codes ``kc``/``vc``
    [W, D] int8, scales ``ks``/``vs`` [W/16] float32, witness ``wit`` [W, D/8]
    float64 (from the stored fp16), slot positions ``pos`` [W], staging rows
    ``ksg``/``vsg`` [16, D] (bf16 bits).  Codes, scales and positions
    bit-exact vs the oracle; the stored witness never below the exact band
    norm and within one fp16 step above it; staging rows equal the inputs."""
    st = decoder.expected_int8_store(k64, v64, n, W)
    np.testing.assert_array_equal(pos, st["slot_pos"], err_msg=f"{what} slot positions")
    live = np.nonzero(st["slot_pos"] >= 0)[0]
    np.testing.assert_array_equal(kc[live], st["k_codes"][live], err_msg=f"{what} key codes")
    np.testing.assert_array_equal(vc[live], st["v_codes"][live], err_msg=f"{what} value codes")
    lb = np.unique(live // 16)
    np.testing.assert_array_equal(ks[lb], st["k_scale"][lb], err_msg=f"{what} key scales")
    np.testing.assert_array_equal(vs[lb], st["v_scale"][lb], err_msg=f"{what} value scales")
    we, wg = st["witness"][live], wit[live]
    assert np.all(wg >= we), f"{what}: stored witness below the exact band norm"
    assert np.all(wg <= we * (1 + 2.0 ** -9) + 2.0 ** -24), f"{what}: stored witness not tight"
    for p in st["staged_positions"]:
        np.testing.assert_array_equal(bits.to_f64(ksg[p % 16]), k64[p])
        np.testing.assert_array_equal(bits.to_f64(vsg[p % 16]), v64[p])


def fp16_witness_slack(q64) -> float:
    """Absolute excess a bound may carry when band norms fall below fp16's
    normal range (6.1e-5): each stored norm, rounded up, may sit one subnormal
    step (2^-24) above the exact one, so c_t may exceed the exact bound by
    sum_b ||q_b|| 2^-24 / sqrt(D)."""
    q64 = np.asarray(q64, dtype=np.float64)
    d = q64.shape[-1]
    return float(np.sum(np.linalg.norm(q64.reshape(-1, 8), axis=1)) * 2.0 ** -24 / np.sqrt(d))


def check_int8_decode(out, cmax, c_all, b, h, q64, k64, v64, n, W, what=""):
    """INT8 decode of (b, h) vs the oracle: output within TOL; cmax and every
    per-slot c_t sound (>= the true logit error of that token) and tight
    (within (1 + 2^-9), plus the fp16 subnormal slack for tiny residuals)."""
    res = oint8.int8_decode(q64, k64, v64, n, W)
    err = assert_close(out, res["out"], f"int8 out {what} b={b} h={h}")
    e, c = res["e"], res["c"]
    slack = fp16_witness_slack(q64) + 1e-30
    emax = float(np.max(e)) if e.size else 0.0
    assert cmax >= emax, f"cmax {cmax} below the true max logit error {emax}"
    assert cmax <= (res["cmax"] + slack) * (1 + 2.0 ** -9), (cmax, res["cmax"])
    if c_all is not None:
        slots = res["positions"] % W
        cg = np.asarray(c_all, dtype=np.float64)[slots]
        assert np.all(cg >= e), "per-token bound below the true logit error"
        assert np.all(cg <= (c + slack) * (1 + 2.0 ** -9)), "per-token bound not tight"
        quant = res["positions"] < 16 * (n // 16)
        assert not np.any(cg[~quant]), "exact (staged) tokens must have c = 0"
        vis = np.zeros(W, dtype=bool)
        vis[slots[quant]] = True
        assert not np.any(np.asarray(c_all)[~vis]), "slots without a visible quantized token must be 0"
    return err


def check_dither_decode(out, cert, b, h, q64, k64, v64, n, W, req, layer, delta, tv=None, gate=None,
                        tau=0.2, what="", position0=0):
    """Tier B decode of (b, h) vs the oracle: output within TOL; the
    certificate equal to the oracle's up to its float32 pad, and (an event of
    probability >= 1 - delta) not below the true largest logit error; tv =
    tanh(cert/2) padded, and gate = tv > tau."""
    res = odither.int8_dither_decode(q64, k64, v64, n, W, req, layer, h, float(np.float32(delta)), position0)
    err = assert_close(out, res["out"], f"dither out {what} b={b} h={h}")
    ref = res["cert"]
    assert cert >= ref, (what, b, h, cert, ref)
    assert cert <= ref * (1 + 2.0 ** -10) + 1e-30, (what, b, h, cert, ref)
    emax = float(np.max(res["e"])) if res["e"].size else 0.0
    assert cert >= emax, f"{what} b={b} h={h}: certificate {cert} below the logit error {emax}"
    if tv is not None:
        t = float(np.tanh(cert / 2))
        assert t <= tv <= min(t * (1 + 2.0 ** -18) + 1e-30, 1.0), (tv, t)
        if gate is not None:
            assert int(gate) == int(tv > tau)
    return err
