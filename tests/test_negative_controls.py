"""Negative controls for the comparisons in the GPU parity tests (CPU only).

The GPU parity tests are only as strong as their comparisons.  Here the
correct state and outputs come from the oracle, a planted mistake of each
class the sliding-window pages warn about (page "用Lean4形式化验证滑动窗口KV
Cache的正确性", §1.2 and §5.1; page "LLM 機制實驗（五）": a stale
next_position) is applied to them on the CPU, and those comparisons must reject
every one: slot off by one, wrong base while the ring fills, stale
next_position, head advanced before the write; for the outputs, a decode
with a stale next_position; for the bounds, a zeroed witness and a halved
certificate.  No GPU code runs.
"""

import numpy as np
import pytest
import torch

from oracle import decoder, dither as odither, int8 as oint8
from tests.gpu_util import assert_close, check_dither_decode, check_int8_decode, check_ring_rows, oracle_out

W, H, D = 6, 2, 16


class Ring:
    """A ring cache state as CPU tensors (the layout the GPU tests read)."""

    def __init__(self, k_bits, v_bits, n, slot_of=lambda p: p % W, pos_of=lambda p: p, np_value=None):
        B = k_bits.shape[0]
        self.B, self.W, self.layout = B, W, "ring"
        self.k = torch.zeros((B, H, W, D), dtype=torch.int16)
        self.v = torch.zeros_like(self.k)
        self.pos = torch.full((B, W), -1, dtype=torch.int32)
        self.next_position = torch.tensor([n if np_value is None else np_value] * B, dtype=torch.int32)
        for b in range(B):
            for p in range(max(0, n - W), n):
                s = slot_of(p)
                self.k[b, :, s] = torch.from_numpy(k_bits[b, :, p].view(np.int16))
                self.v[b, :, s] = torch.from_numpy(v_bits[b, :, p].view(np.int16))
                self.pos[b, s] = pos_of(p)
        self.k, self.v = self.k.view(torch.bfloat16), self.v.view(torch.bfloat16)  # bf16 rows, as on the GPU


def data(n, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 1 << 16, size=(1, H, n, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(1, H, n, D), dtype=np.uint16)
    return k, v


@pytest.mark.parametrize("n", [3, 6, 7, 13])
def test_correct_ring_passes(n):
    k, v = data(n)
    check_ring_rows(Ring(k, v, n), k, v, np.array([n]))


@pytest.mark.parametrize("n", [3, 6, 7, 13])
def test_slot_off_by_one_is_caught(n):
    k, v = data(n)
    bad = Ring(k, v, n, slot_of=lambda p: (p + 1) % W)
    with pytest.raises(AssertionError):
        check_ring_rows(bad, k, v, np.array([n]))


def test_wrong_base_while_filling_is_caught():
    n = 4  # unfilled: the first token must sit in slot 0
    k, v = data(n)
    bad = Ring(k, v, n, slot_of=lambda p: (p + W - 1) % W)
    with pytest.raises(AssertionError):
        check_ring_rows(bad, k, v, np.array([n]))


@pytest.mark.parametrize("n", [4, 6, 9])
def test_stale_next_position_is_caught(n):
    k, v = data(n)
    with pytest.raises(AssertionError):
        check_ring_rows(Ring(k, v, n, np_value=n - 1), k, v, np.array([n]))


@pytest.mark.parametrize("n", [7, 12])
def test_head_advanced_before_the_write_is_caught(n):
    # the newest token's slot still holds the token it should have evicted
    k, v = data(n)
    bad = Ring(k, v, n)
    s = (n - 1) % W
    old = n - 1 - W
    bad.k[0, :, s] = torch.from_numpy(k[0, :, old].view(np.int16)).view(torch.bfloat16)
    bad.v[0, :, s] = torch.from_numpy(v[0, :, old].view(np.int16)).view(torch.bfloat16)
    bad.pos[0, s] = old
    with pytest.raises(AssertionError):
        check_ring_rows(bad, k, v, np.array([n]))


@pytest.mark.parametrize("seed", range(4))
def test_decode_with_stale_next_position_is_caught(seed):
    rng = np.random.default_rng(seed)
    n, w = 40, 16
    k = rng.standard_normal((H, n, D))
    v = rng.standard_normal((H, n, D))
    q = rng.standard_normal((H, D))
    good = oracle_out(k, v, q, n, w)
    stale = oracle_out(k, v, q, n - 1, w)  # attends to the window one step back
    assert_close(good, good, "control")
    with pytest.raises(AssertionError):
        assert_close(stale, good, "stale next_position")


def test_zeroed_witness_is_caught():
    rng = np.random.default_rng(3)
    n, w = 60, 32
    k = rng.standard_normal((n, 128))
    v = rng.standard_normal((n, 128))
    q = rng.standard_normal(128)
    res = oint8.int8_decode(q, k, v, n, w)
    check_int8_decode(res["out"], res["cmax"], None, 0, 0, q, k, v, n, w)   # the oracle's own bound passes
    with pytest.raises(AssertionError):
        check_int8_decode(res["out"], 0.0, None, 0, 0, q, k, v, n, w)      # a zeroed witness gives cmax = 0


def test_halved_certificate_is_caught():
    rng = np.random.default_rng(4)
    n, w = 60, 32
    k = rng.standard_normal((n, 128)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((n, 128)).astype(np.float32).astype(np.float64)
    q = rng.standard_normal(128)
    delta = float(np.float32(1e-3))
    res = odither.int8_dither_decode(q, k, v, n, w, 9, 0, 0, delta)
    cert = res["cert"] * (1 + 2.0 ** -12)
    check_dither_decode(res["out"], cert, 0, 0, q, k, v, n, w, 9, 0, 1e-3)
    with pytest.raises(AssertionError):
        check_dither_decode(res["out"], 0.5 * cert, 0, 0, q, k, v, n, w, 9, 0, 1e-3)
