"""Synthetic decode workloads: shapes, sizes and seeds.

Each entry is one workload of the sliding-window decode step, named by what
it is.  The numbers restate the workload table the benchmark and the parity
tests share; ``gen`` turns an entry into seeded input tensors.  Nothing here
computes any part of the decode step.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class Workload:
    cid: int                 # seed namespace
    name: str
    kind: str                # "fp32" | "bf16" | "int8" | "int8_dither"
    B: int
    H: int
    D: int
    W: int                   # window = ring capacity in tokens
    prefill: int = 0         # tokens appended before the first timed/checked query
    steps: int = 0           # decode steps (append one token, then attend)
    ragged: Optional[tuple] = None   # inclusive (lo, hi) per-sequence lengths
    spike_frac: float = 0.0  # fraction of keys per (b, h) multiplied by spike_mul
    spike_mul: float = 8.0
    rope_base: Optional[float] = None
    prefill_chunk: int = 0   # 0 = one chunk
    layout: str = "ring"     # "ring" | "paged" (16-token pages through a block table)
    note: str = field(default="", compare=False)


TINY = Workload(1, "tiny-window4-fp32", "fp32", B=1, H=2, D=16, W=4, prefill=0, steps=12,
                note="12 decode steps from an empty cache: unfilled, exactly full, overwrite")
FULL_RAGGED = Workload(2, "full-cache-ragged-4096-bf16", "bf16", B=8, H=32, D=128, W=4096,
                       ragged=(1024, 4096),
                       note="no window (W = capacity), ragged lengths U{1024..4096}")
RING = Workload(3, "ring-w4096-pos8192-bf16", "bf16", B=16, H=32, D=128, W=4096,
                prefill=8192, steps=256, prefill_chunk=4096,
                note="prefill positions 0..8191, then 256 append+attend steps at 8192..8447")
LONG = Workload(4, "long-ctx-131072-bf16", "bf16", B=4, H=8, D=128, W=131072, prefill=131072,
                spike_frac=0.01, spike_mul=8.0,
                note="1% of keys per (b,h) scaled x8 for a peaked softmax")
INT8_32K = Workload(5, "int8-witness-ctx32768", "int8", B=16, H=32, D=128, W=32768,
                    prefill=32768, steps=20, rope_base=10000.0, prefill_chunk=8192,
                    note="RoPE keys, INT8 per 16-token block, 16-band fp16 witness")
BF16_32K = Workload(6, "bf16-ctx32768", "bf16", B=16, H=32, D=128, W=32768, prefill=32768,
                    rope_base=10000.0, prefill_chunk=8192,
                    note="bf16 companion of the INT8 32k workload")

# Same inputs as the ring workloads above (same seed namespace), paged storage.
INT8_32K_PAGED = Workload(5, "int8-witness-ctx32768-paged", "int8", B=16, H=32, D=128, W=32768,
                          prefill=32768, steps=20, rope_base=10000.0, prefill_chunk=8192, layout="paged",
                          note="the INT8 32k workload in 16-token pages")
BF16_32K_PAGED = Workload(6, "bf16-ctx32768-paged", "bf16", B=16, H=32, D=128, W=32768, prefill=32768,
                          rope_base=10000.0, prefill_chunk=8192, layout="paged",
                          note="the bf16 32k workload in 16-token pages")

# Same inputs as the INT8 32k workload, stored with subtractive dither and no witness.
INT8_DITHER_32K = Workload(5, "int8-dither-ctx32768", "int8_dither", B=16, H=32, D=128, W=32768,
                           prefill=32768, steps=20, rope_base=10000.0, prefill_chunk=8192,
                           note="the INT8 32k workload with Philox subtractive dither (Tier B)")

# One GPU's share when a workload is spread over 8 GPUs (the kernels at a
# shard's real shape; the cross-GPU exchange itself is not built).
LONG_CTX_SHARD = Workload(7, "long-ctx-131072-bf16-ctx-shard-1of8", "bf16", B=4, H=8, D=128, W=16384,
                          prefill=16384, spike_frac=0.01, spike_mul=8.0,
                          note="one GPU's 16384 slots of the 131072 context split 8 ways")
INT8_HEAD_SHARD = Workload(8, "int8-witness-ctx32768-head-shard-1of8", "int8", B=16, H=4, D=128, W=32768,
                           prefill=32768, steps=20, rope_base=10000.0, prefill_chunk=8192,
                           note="one GPU's 4 of the 32 heads of the INT8 32k workload split 8 ways")

ALL = {w.name: w for w in (TINY, FULL_RAGGED, RING, LONG, INT8_32K, BF16_32K, INT8_32K_PAGED, BF16_32K_PAGED,
                           INT8_DITHER_32K, LONG_CTX_SHARD, INT8_HEAD_SHARD)}
