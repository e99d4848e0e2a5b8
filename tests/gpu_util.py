"""Helpers for the GPU parity tests: device checks, host copies of device
tensors, and comparisons of the HIP results with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import bits, decoder, dither as odither
from tests.parity_checks import (TOL, assert_close, check_dither_decode, check_int8_decode,  # noqa: F401
                                 check_int8_store_arrays, fp16_witness_slack, oracle_out)

def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sliding_window_attention_ring_amd as swa
    swa.lib()  # fails loudly if the HIP library is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy with the storage bits: bf16/fp16 -> uint16, others as is."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16/fp32 tensor (host)."""
    return bits.to_f64(host_bits(t))


class RingView:
    """A cache's storage in ring layout: the tensors themselves for a ring
    cache, gathered through the block table for a paged one."""

    def __init__(self, cache):
        self.B, self.H, self.W, self.kind = cache.B, cache.H, cache.W, cache.kind
        self.pos, self.next_position = cache.pos, cache.next_position
        self.k_stage, self.v_stage = cache.k_stage, cache.v_stage
        if cache.layout == "ring":
            self.k, self.v = cache.k, cache.v
            self.k_scale, self.v_scale, self.witness = cache.k_scale, cache.v_scale, cache.witness
            return
        tbl = cache.block_table.long()                       # [B, W/16]
        slots = torch.arange(cache.W, device=tbl.device)
        pages = tbl[:, slots // 16]                          # [B, W]
        rows = (slots % 16).expand_as(pages)

        def gather(pool):                                    # [P, H, 16, X] -> [B, H, W, X]
            return pool[pages, :, rows].permute(0, 2, 1, 3).contiguous()

        self.k, self.v = gather(cache.k), gather(cache.v)
        self.k_scale = self.v_scale = self.witness = None
        if cache.kind in ("int8", "int8_dither"):
            self.k_scale = cache.k_scale[tbl].permute(0, 2, 1).contiguous()  # [B, H, W/16]
            self.v_scale = cache.v_scale[tbl].permute(0, 2, 1).contiguous()
        if cache.kind == "int8":
            self.witness = gather(cache.witness)


def check_ring_rows(cache, k_in: np.ndarray, v_in: np.ndarray, n: np.ndarray):
    """bf16/fp32 cache: pos, next_position and every live slot's K/V bits equal
    what the ring must hold after n[b] appends of rows k_in[b][h][p] (bits)."""
    if not isinstance(cache, RingView) and getattr(cache, "layout", "ring") == "paged":
        cache = RingView(cache)
    pos = host_bits(cache.pos)
    npos = host_bits(cache.next_position)
    kk, vv = host_bits(cache.k), host_bits(cache.v)
    for b in range(cache.B):
        assert npos[b] == n[b], (b, npos[b], n[b])
        exp = decoder.expected_ring(np.arange(n[b]), cache.W)
        np.testing.assert_array_equal(pos[b], exp)
        live = np.nonzero(exp >= 0)[0]
        np.testing.assert_array_equal(kk[b][:, live], k_in[b][:, exp[live]])
        np.testing.assert_array_equal(vv[b][:, live], v_in[b][:, exp[live]])


def check_int8_store(cache, b: int, h: int, k64: np.ndarray, v64: np.ndarray, n: int):
    """INT8 cache of (b, h) against the oracle (check_int8_store_arrays):
    the cache's host copies, read back through the table when paged."""
    if getattr(cache, "layout", "ring") == "paged":
        cache = RingView(cache)
    check_int8_store_arrays(host_bits(cache.k[b, h]), host_bits(cache.v[b, h]), host_bits(cache.k_scale[b, h]),
                            host_bits(cache.v_scale[b, h]),
                            host_bits(cache.witness[b, h]).view(np.float16).astype(np.float64),
                            host_bits(cache.pos[b]), host_bits(cache.k_stage[b, h]), host_bits(cache.v_stage[b, h]),
                            k64, v64, n, cache.W, f"b={b} h={h}")


def request_ids(cache) -> np.ndarray:
    """The cache's request ids as Python ints (uint64 values)."""
    return [int(x) & ((1 << 64) - 1) for x in cache.request_id.cpu().tolist()]


def check_dither_store(cache, b: int, h: int, k64: np.ndarray, v64: np.ndarray, n: int, position0: int = 0,
                       first_block: int = 0):
    """Tier B cache of (b, h): slot positions, codes and scales of every
    committed block in the ring bit-exact vs the oracle (which draws the same
    Philox dither itself); staging rows equal the input bits.  Row j of the
    history has position position0 + j (position0 a multiple of W); blocks
    below first_block are not compared (their codes may predate position0)."""
    req, layer = request_ids(cache)[b], cache.layer
    view = RingView(cache) if getattr(cache, "layout", "ring") == "paged" else cache
    W = cache.W
    nb = n // 16
    pos = host_bits(view.pos[b])
    kc = host_bits(view.k[b, h]); vc = host_bits(view.v[b, h])
    ks = host_bits(view.k_scale[b, h]); vs = host_bits(view.v_scale[b, h])
    exp_pos = np.full(W, -1, dtype=np.int64)
    for kb in range(max(0, nb - W // 16), nb):
        rows = np.arange(kb * 16, kb * 16 + 16)
        exp_pos[(kb * 16) % W:(kb * 16) % W + 16] = rows + position0
        if kb < first_block:
            continue
        u = odither.dither(req, layer, h, rows + position0, k64.shape[-1])
        sk, ck = odither.quantize_block(k64[rows], u)
        sv, cv = odither.quantize_block(v64[rows], u)
        slot0 = (kb * 16) % W
        np.testing.assert_array_equal(kc[slot0:slot0 + 16], ck, err_msg=f"key codes b={b} h={h} block {kb}")
        np.testing.assert_array_equal(vc[slot0:slot0 + 16], cv, err_msg=f"value codes b={b} h={h} block {kb}")
        assert ks[slot0 // 16] == sk and vs[slot0 // 16] == sv, (kb, ks[slot0 // 16], sk)
    np.testing.assert_array_equal(pos, exp_pos)
    ksg = host_bits(cache.k_stage[b, h]); vsg = host_bits(cache.v_stage[b, h])
    for p in range(16 * nb, n):
        np.testing.assert_array_equal(bits.to_f64(ksg[p % 16]), k64[p])
        np.testing.assert_array_equal(bits.to_f64(vsg[p % 16]), v64[p])
