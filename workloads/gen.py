"""Seeded synthetic inputs for the decode workloads.

Only random numbers and input preparation live here: normal draws, rounding
to the storage dtype (torch's round-to-nearest-even cast to bfloat16), ragged
lengths, which keys get spiked, and rotary rotation of the inputs.  Both the
HIP path and the CPU oracle consume exactly the tensors produced here, so
they see identical bits.  Nothing here computes any part of the decode step.

Seeds: every tensor draws from its own stream, seeded from
``(2026, workload id, tensor name, index...)``; per-sequence tensors are
seeded per sequence so a result does not depend on how generation is chunked.
"""

from __future__ import annotations

import zlib
from typing import Optional, Sequence

import numpy as np
import torch


def seed(cid: int, name: str, *extra: int) -> int:
    ss = np.random.SeedSequence([2026, int(cid), zlib.crc32(name.encode()), *map(int, extra)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> 1)


def normal(shape: Sequence[int], s: int, device="cpu") -> torch.Tensor:
    """float32 N(0, 1) draws from torch's generator for ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)


def storage_dtype(kind: str) -> torch.dtype:
    return torch.float32 if kind == "fp32" else torch.bfloat16


def tokens(wl, which: str, n: int, device="cpu", b_range: Optional[range] = None) -> torch.Tensor:
    """Key or value rows ``[B, H, n, D]`` for positions ``0 .. n-1``.

    ``which`` is "k" or "v".  Keys of a workload with ``spike_frac`` get that
    fraction of rows per (b, h) multiplied by ``spike_mul`` (exact in bf16 for
    a power of two).  Keys of a workload with ``rope_base`` are rotated at
    their absolute positions (interleaved pairs) before rounding; values are
    never rotated.
    """
    b_range = range(wl.B) if b_range is None else b_range
    out = torch.empty((len(b_range), wl.H, n, wl.D), dtype=storage_dtype(wl.kind), device=device)
    cos = sin = None
    if wl.rope_base is not None and which == "k":
        cos, sin = rope_tables(np.arange(n), wl.D, wl.rope_base, device)
    for i, b in enumerate(b_range):
        x = normal((wl.H, n, wl.D), seed(wl.cid, which, b), device)
        if cos is not None:
            x = rope_rotate(x, cos, sin)
        if wl.spike_frac and which == "k":
            for h in range(wl.H):
                rows = spike_rows(wl, b, h, n)
                x[h, torch.as_tensor(rows, device=device)] *= wl.spike_mul
        out[i] = x.to(out.dtype)
    return out


def query(wl, step_pos: int, device="cpu") -> torch.Tensor:
    """Query ``[B, H, D]`` of the decode step at absolute position ``step_pos``."""
    x = normal((wl.B, wl.H, wl.D), seed(wl.cid, "q", step_pos), device)
    if wl.rope_base is not None:
        cos, sin = rope_tables(np.array([step_pos]), wl.D, wl.rope_base, device)
        x = rope_rotate(x.unsqueeze(2), cos, sin).squeeze(2)
    return x.to(storage_dtype(wl.kind))


def ragged_lengths(wl) -> np.ndarray:
    """Per-sequence lengths, integer uniform on ``wl.ragged`` inclusive."""
    lo, hi = wl.ragged
    rng = np.random.Generator(np.random.PCG64(seed(wl.cid, "len")))
    return rng.integers(lo, hi + 1, size=wl.B).astype(np.int64)


def spike_rows(wl, b: int, h: int, n: int) -> np.ndarray:
    """``round(spike_frac * n)`` distinct positions, uniform, for (b, h)."""
    cnt = int(round(wl.spike_frac * n))
    rng = np.random.Generator(np.random.PCG64(seed(wl.cid, "spike", b, h)))
    return np.sort(rng.choice(n, size=cnt, replace=False))


def rope_tables(positions: np.ndarray, d: int, base: float, device="cpu"):
    """cos/sin ``[n, D/2]`` (angles in float64, stored float32)."""
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * base ** (-2.0 * i / d)
    return (torch.from_numpy(np.cos(ang).astype(np.float32)).to(device),
            torch.from_numpy(np.sin(ang).astype(np.float32)).to(device))


def rope_rotate(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Rotate interleaved pairs of ``x [..., n, D]`` (float32)."""
    a, b = x[..., 0::2], x[..., 1::2]
    y = torch.empty_like(x)
    y[..., 0::2] = a * cos - b * sin
    y[..., 1::2] = a * sin + b * cos
    return y


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as uint16 bit patterns (fp32 -> float32 array)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()
