"""Philox-4xW counter-based generator (the generator [WitCert] names for Tier B).

Follows the published definition: J. K. Salmon, M. A. Moraes, R. O. Dror,
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011), the
Philox family.  A 4-word counter ``(x0, x1, x2, x3)`` and a 2-word key
``(k0, k1)`` of W-bit words go through R rounds; each round

* multiplies ``x0`` by ``M0`` and ``x2`` by ``M1`` into double-width products
  and splits each into its high and low W-bit halves;
* outputs ``(hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0))``;
* then bumps the key by the Weyl constants: ``k0 += C0``, ``k1 += C1`` (mod 2^W).

The first round uses the key as given.  The constants are the paper's:
W = 32: M0 = 0xD2511F53, M1 = 0xCD9E8D57, C0 = 0x9E3779B9 (golden ratio),
C1 = 0xBB67AE85 (sqrt(3) - 1); W = 64: M0 = 0xD2E7470EE14C6C93,
M1 = 0xCA5A826395121157, C0 = 0x9E3779B97F4A7C15, C1 = 0xBB67AE8584CAA73B.
Ten rounds is the recommended (default) count.

Two forms: ``philox`` (plain Python integers, any width) and
``philox4x32`` (NumPy, vectorized over many counters, W = 32 only).

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np

_CONST = {
    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85),
    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),
}
ROUNDS = 10


def philox(counter, key, width: int = 32, rounds: int = ROUNDS) -> tuple:
    """Philox-4x``width``-``rounds`` of one counter; returns 4 words (ints)."""
    m0, m1, c0, c1 = _CONST[width]
    mask = (1 << width) - 1
    x0, x1, x2, x3 = (int(v) & mask for v in counter)
    k0, k1 = (int(v) & mask for v in key)
    for _ in range(rounds):
        p0 = m0 * x0
        p1 = m1 * x2
        x0, x1, x2, x3 = ((p1 >> width) ^ x1 ^ k0, p1 & mask, (p0 >> width) ^ x3 ^ k1, p0 & mask)
        k0 = (k0 + c0) & mask
        k1 = (k1 + c1) & mask
    return (x0, x1, x2, x3)


def philox4x32(counter: np.ndarray, key: np.ndarray, rounds: int = ROUNDS) -> np.ndarray:
    """Philox-4x32 over arrays: ``counter`` [..., 4], ``key`` [..., 2] (broadcast).

    Returns uint32 [..., 4].  The 32x32-bit products are formed exactly in
    uint64.
    """
    m0, m1, c0, c1 = (np.uint64(v) for v in _CONST[32])
    lo32 = np.uint64(0xFFFFFFFF)
    sh = np.uint64(32)
    ctr = np.asarray(counter, dtype=np.uint64) & lo32
    k = np.asarray(key, dtype=np.uint64) & lo32
    x0, x1, x2, x3 = (ctr[..., i] for i in range(4))
    k0, k1 = k[..., 0], k[..., 1]
    for _ in range(rounds):
        p0 = m0 * x0
        p1 = m1 * x2
        x0, x1, x2, x3 = ((p1 >> sh) ^ x1 ^ k0, p1 & lo32, (p0 >> sh) ^ x3 ^ k1, p0 & lo32)
        k0 = (k0 + c0) & lo32
        k1 = (k1 + c1) & lo32
    return np.stack(np.broadcast_arrays(x0, x1, x2, x3), axis=-1).astype(np.uint32)
