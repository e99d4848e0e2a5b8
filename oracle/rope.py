"""Rotary position embedding, float64, for the band-unitarity check.

[WitCert] "频带酉性与双层证书" section: RoPE is a block-diagonal orthogonal map
over frequency pairs, so for every contiguous band ``b`` that is a union of
whole rotation pairs and every shift ``n``, ``||(R_n x)_b|| = ||x_b||``.

Reading taken (the pages do not fix the pairing): interleaved pairs
``(2i, 2i+1)`` with frequency ``theta_i = base^(-2i/D)`` and angle
``pos * theta_i``.  Each 8-dim band then holds four whole pairs.  The
half-split pairing ``(i, i + D/2)`` is provided only to show that the band
identity fails for it.

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np


def _angles(pos: np.ndarray, d: int, base: float) -> np.ndarray:
    i = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta  # [..., D/2]


def rope_interleaved(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate pairs ``(x[2i], x[2i+1])`` by ``pos * theta_i`` (float64)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = _angles(np.broadcast_to(pos, x.shape[:-1]), d, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def rope_half_split(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate pairs ``(x[i], x[i + D/2])`` by ``pos * theta_i`` (float64)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = _angles(np.broadcast_to(pos, x.shape[:-1]), d, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
