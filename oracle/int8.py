"""INT8 block quantization of the KV cache and the band-norm witness bound.

Follows [WitCert]:
* "频带酉性与双层证书" section: features split into contiguous bands; the
  witness ``w_{t,b}`` is the Euclidean norm of band ``b`` of the quantization
  residual ``r_t`` of the key, recorded when the token is written; the
  logit error ``|eps_t| = |q . r_t| / sqrt(d)`` is bounded by
  ``c_t = (1/sqrt(d)) * sum_b ||q_b|| * w_{t,b}`` (Cauchy-Schwarz per band,
  then the triangle inequality); 16 bands, 32 bytes per token per head.
* "SGLang 生产级落地" section: one scale per block, so the scale is a scalar
  independent of the token inside the block.

Readings taken where the pages are silent:
* Blocks are 16 consecutive absolute positions aligned at ``pos // 16``;
  one float32 absmax scale per (sequence, head, block) per tensor, symmetric
  codes in [-127, 127].  The scale and code steps are fixed in float32:
  ``s = f32(f32(max|x|) / f32(127))`` and ``code = rint(f32(x) / s)`` with IEEE
  division and round-half-to-even, clamped to +-127; ``s == 0`` gives all-zero
  codes.
* Bands are consecutive groups of ``band = 8`` dimensions (16 bands at
  D = 128, the pages' setting).
* The "true" key is the input key the unquantized cache would hold; the
  residual is ``k - s * code`` evaluated exactly (float64).
* Only complete blocks are quantized; the newest ``next_position mod 16``
  tokens stay exact and carry ``c_t = 0``.
* V is quantized the same way; the bound covers logit error only, so V has
  no witness.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from .attention import softmax_weights

BLOCK = 16
BAND = 8
QMAX = 127


def block_scale(x: np.ndarray) -> np.float32:
    """float32 absmax scale of one block: ``f32(f32(max|x|) / f32(127))``."""
    x32 = np.asarray(x, dtype=np.float32)
    a = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    return np.float32(a / np.float32(QMAX))


def block_codes(x: np.ndarray, s: np.float32) -> np.ndarray:
    """Codes ``clamp(rint(f32(x) / s), -127, 127)`` as int8 (zeros if s == 0)."""
    x32 = np.asarray(x, dtype=np.float32)
    if s == 0:
        return np.zeros(x32.shape, dtype=np.int8)
    q = np.rint(x32 / np.float32(s))  # float32 IEEE division, half-to-even
    return np.clip(q, -QMAX, QMAX).astype(np.int8)


def quantize_block(x: np.ndarray):
    """Quantize one ``[16, D]`` block -> (scale float32, codes int8 [16, D])."""
    s = block_scale(x)
    return s, block_codes(x, s)


def dequantize(codes: np.ndarray, s) -> np.ndarray:
    """``s * code`` in float64 (exact: a float32 times an 8-bit integer)."""
    return np.float64(np.float32(s)) * np.asarray(codes, dtype=np.float64)


def band_norms(x: np.ndarray, band: int = BAND) -> np.ndarray:
    """Euclidean norm of each contiguous band of ``band`` dims (last axis)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % band == 0
    xb = x.reshape(x.shape[:-1] + (d // band, band))
    return np.sqrt(np.sum(xb * xb, axis=-1))


def logit_error(q: np.ndarray, r: np.ndarray) -> np.ndarray:
    """True logit error ``|q . r_t| / sqrt(d)`` for rows ``r`` ([WitCert])."""
    q = np.asarray(q, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return np.abs(r @ q) / np.sqrt(q.shape[-1])


def witness_bound(q: np.ndarray, w: np.ndarray, band: int = BAND) -> np.ndarray:
    """``c_t = (1/sqrt(d)) sum_b ||q_b|| w_{t,b}`` for witness rows ``w``."""
    q = np.asarray(q, dtype=np.float64)
    nq = band_norms(q, band)
    return (np.asarray(w, dtype=np.float64) @ nq) / np.sqrt(q.shape[-1])


def quantize_history(x: np.ndarray, n_complete_blocks: int):
    """Quantize the first ``n_complete_blocks`` blocks of a history ``[n, D]``.

    Returns (scales float32 [nb], codes int8 [nb*16, D]).
    """
    x = np.asarray(x)
    nb = n_complete_blocks
    scales = np.zeros(nb, dtype=np.float32)
    codes = np.zeros((nb * BLOCK, x.shape[-1]), dtype=np.int8)
    for blk in range(nb):
        rows = slice(blk * BLOCK, (blk + 1) * BLOCK)
        s, c = quantize_block(x[rows])
        scales[blk] = s
        codes[rows] = c
    return scales, codes


def int8_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, next_position: int,
                w: int, band: int = BAND) -> dict:
    """One INT8 decode query over a history whose row ``j`` has position ``j``.

    The query is at step ``t = next_position - 1`` and sees positions
    ``[t - len + 1, t]`` with ``len = min(w, next_position)``.  Tokens in
    complete blocks (``pos < 16 * (next_position // 16)``) are read
    dequantized; the newer ones are exact.  Returns float64 ``out``, the
    visible positions, and per visible token the bound ``c`` (0 for exact
    tokens), the true logit error ``e`` and the exact witness rows ``wit``;
    plus ``cmax = max c`` (0 if nothing is visible).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = next_position
    assert k.shape[0] >= n and v.shape[0] >= n
    d = q.shape[-1]
    nb = n // BLOCK
    nq = nb * BLOCK
    ks, kc = quantize_history(k[:nq], nb)
    vs, vc = quantize_history(v[:nq], nb)
    k_hat = k[:n].copy()
    v_hat = v[:n].copy()
    for blk in range(nb):
        rows = slice(blk * BLOCK, (blk + 1) * BLOCK)
        k_hat[rows] = dequantize(kc[rows], ks[blk])
        v_hat[rows] = dequantize(vc[rows], vs[blk])
    r = k[:n] - k_hat  # exact residual; zero for the exact (newest) tokens
    t = n - 1
    ln = min(w, n)
    vis = np.arange(t - ln + 1, t + 1, dtype=np.int64)
    wit = band_norms(r[vis], band)
    c = witness_bound(q, wit, band)
    e = logit_error(q, r[vis])
    if ln == 0:
        out = np.zeros(v.shape[-1], dtype=np.float64)
    else:
        out = softmax_weights((k_hat[vis] @ q) / np.sqrt(d)) @ v_hat[vis]
    return {
        "out": out,
        "positions": vis,
        "c": c,
        "e": e,
        "wit": wit,
        "cmax": float(np.max(c)) if ln else 0.0,
        "k_scales": ks,
        "v_scales": vs,
        "k_codes": kc,
        "v_codes": vc,
    }
