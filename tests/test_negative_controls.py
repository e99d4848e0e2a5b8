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
from tests.gpu_util import (assert_close, check_dither_decode, check_dither_store, check_int8_decode, check_ring_rows,
                            oracle_out)
from tests.parity_checks import check_int8_store_arrays

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


# Each assertion of the INT8, Tier B and ring comparisons rejects a state or
# output that differs from the oracle's in that one respect.  The "GPU"
# state is built from the oracle the way the kernels store it (witness
# rounded up to fp16, bounds padded), the comparison must accept it, and
# each planted difference must be rejected.

def _bf16_rows(rng, n, d):
    """n rows of bf16 bit patterns (finite) and their float64 values."""
    f32 = rng.standard_normal((n, d)).astype(np.float32)
    bits16 = (f32.view(np.uint32) >> 16).astype(np.uint16)
    return bits16, (bits16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _fp16_up(x):
    """Nonnegative float64 -> nearest fp16 at or above it, as float64."""
    h = x.astype(np.float16)
    below = h.astype(np.float64) < x
    h[below] = np.nextafter(h[below], np.float16(np.inf))
    return h.astype(np.float64)


class Int8State:
    def __init__(self, n=16 * 5 + 7, w=48, seed=5):
        rng = np.random.default_rng(seed)
        self.n, self.w = n, w
        self.kbits, self.k64 = _bf16_rows(rng, n, 128)
        self.vbits, self.v64 = _bf16_rows(rng, n, 128)
        st = decoder.expected_int8_store(self.k64, self.v64, n, w)
        self.kc, self.vc = st["k_codes"].copy(), st["v_codes"].copy()
        self.ks, self.vs = st["k_scale"].copy(), st["v_scale"].copy()
        self.exact_wit = st["witness"]
        self.wit = _fp16_up(st["witness"])
        self.pos = st["slot_pos"].copy()
        self.ksg = np.zeros((16, 128), dtype=np.uint16)
        self.vsg = np.zeros((16, 128), dtype=np.uint16)
        self.staged = st["staged_positions"]
        for p in self.staged:
            self.ksg[p % 16], self.vsg[p % 16] = self.kbits[p], self.vbits[p]
        self.live = np.nonzero(self.pos >= 0)[0]

    def check(self):
        check_int8_store_arrays(self.kc, self.vc, self.ks, self.vs, self.wit, self.pos, self.ksg, self.vsg,
                                self.k64, self.v64, self.n, self.w)


def test_int8_store_comparison_accepts_the_oracle_state():
    Int8State().check()


@pytest.mark.parametrize("field", ["witness_below", "witness_loose", "k_codes", "v_codes", "k_scale", "v_scale",
                                   "k_stage", "v_stage", "pos"])
def test_int8_store_comparison_rejects_each_field(field):
    s = Int8State()
    slot = s.live[len(s.live) // 2]
    if field == "witness_below":
        # one band rounded down instead of up: below the exact norm
        b = int(np.argmax(s.wit[slot] > s.exact_wit[slot]))
        s.wit[slot, b] = np.nextafter(np.float16(s.wit[slot, b]), np.float16(0)).astype(np.float64)
        assert s.wit[slot, b] < s.exact_wit[slot, b]
    elif field == "witness_loose":
        s.wit[slot, 3] *= 1.01
    elif field == "k_codes":
        s.kc[slot, 7] += 1 if s.kc[slot, 7] < 127 else -1
    elif field == "v_codes":
        s.vc[slot, 7] += 1 if s.vc[slot, 7] < 127 else -1
    elif field == "k_scale":
        s.ks[slot // 16] = np.nextafter(s.ks[slot // 16], np.float32(np.inf))
    elif field == "v_scale":
        s.vs[slot // 16] = np.nextafter(s.vs[slot // 16], np.float32(np.inf))
    elif field == "k_stage":
        s.ksg[s.staged[-1] % 16, 5] ^= 1
    elif field == "v_stage":
        s.vsg[s.staged[-1] % 16, 5] ^= 1
    elif field == "pos":
        s.pos[slot] += s.w  # same slot, the wrong absolute position
    with pytest.raises(AssertionError):
        s.check()


class Int8Decode:
    def __init__(self, n=16 * 3 + 9, w=64, seed=8):
        rng = np.random.default_rng(seed)
        self.n, self.w = n, w
        self.k64 = rng.standard_normal((n, 128))
        self.v64 = rng.standard_normal((n, 128))
        self.q64 = rng.standard_normal(128)
        res = oint8.int8_decode(self.q64, self.k64, self.v64, n, w)
        self.res = res
        self.out = res["out"].copy()
        self.cmax = res["cmax"] * (1 + 2.0 ** -12)
        self.quant = res["positions"] < 16 * (n // 16)
        self.slots = res["positions"] % w
        self.c_all = np.zeros(w)
        self.c_all[self.slots[self.quant]] = res["c"][self.quant] * (1 + 2.0 ** -12)

    def check(self):
        check_int8_decode(self.out, self.cmax, self.c_all, 0, 0, self.q64, self.k64, self.v64, self.n, self.w)


def test_int8_decode_comparison_accepts_the_oracle_outputs():
    Int8Decode().check()


@pytest.mark.parametrize("field", ["out", "cmax_loose", "c_below_error", "c_loose", "c_on_staged", "c_on_empty_slot"])
def test_int8_decode_comparison_rejects_each_output(field):
    d = Int8Decode()
    assert d.n < d.w and not d.quant.all()   # unwritten slots and staged tokens exist
    t = int(np.argmax(np.where(d.quant, d.res["e"], -1)))   # the quantized token with the largest error
    if field == "out":
        d.out[3] += 4e-3
    elif field == "cmax_loose":
        d.cmax *= 1.01
    elif field == "c_below_error":
        d.c_all[d.slots[t]] = d.res["e"][t] * 0.99
    elif field == "c_loose":
        d.c_all[d.slots[t]] *= 1.01
    elif field == "c_on_staged":
        d.c_all[d.slots[~d.quant][0]] = 0.1
    elif field == "c_on_empty_slot":
        d.c_all[d.w - 1] = 0.1
    with pytest.raises(AssertionError):
        d.check()


class DitherDecode:
    def __init__(self, n=60, w=32, seed=4, tau=0.2):
        rng = np.random.default_rng(seed)
        self.n, self.w, self.tau = n, w, tau
        self.k64 = rng.standard_normal((n, 128)).astype(np.float32).astype(np.float64)
        self.v64 = rng.standard_normal((n, 128)).astype(np.float32).astype(np.float64)
        self.q64 = rng.standard_normal(128)
        self.delta = 1e-3
        res = odither.int8_dither_decode(self.q64, self.k64, self.v64, n, w, 9, 0, 0,
                                         float(np.float32(self.delta)))
        self.out = res["out"].copy()
        self.cert = res["cert"] * (1 + 2.0 ** -12)
        self.tv = min(float(np.tanh(self.cert / 2)) * (1 + 2.0 ** -20), 1.0)
        self.gate = int(self.tv > tau)

    def check(self):
        check_dither_decode(self.out, self.cert, 0, 0, self.q64, self.k64, self.v64, self.n, self.w, 9, 0,
                            self.delta, self.tv, self.gate, tau=self.tau)


def test_dither_decode_comparison_accepts_the_oracle_outputs():
    DitherDecode().check()


@pytest.mark.parametrize("field", ["out", "cert_loose", "tv_below", "tv_loose", "gate"])
def test_dither_decode_comparison_rejects_each_output(field):
    d = DitherDecode()
    if field == "out":
        d.out[0] -= 4e-3
    elif field == "cert_loose":  # with tv and gate consistent with it, so only the tightness check can object
        d.cert *= 1.01
        d.tv = min(float(np.tanh(d.cert / 2)) * (1 + 2.0 ** -20), 1.0)
        d.gate = int(d.tv > d.tau)
    elif field == "tv_below":
        d.tv *= 1 - 1e-4
    elif field == "tv_loose":
        d.tv *= 1 + 1e-4
    elif field == "gate":
        d.gate = 1 - d.gate
    with pytest.raises(AssertionError):
        d.check()


def test_ring_comparison_rejects_a_wrong_position_record():
    """Rows in the right slots, but a slot's recorded absolute position is off
    by the window (the same slot, another lap)."""
    n = 9
    k, v = data(n)
    bad = Ring(k, v, n)
    bad.pos[0, (n - 1) % W] += W
    with pytest.raises(AssertionError):
        check_ring_rows(bad, k, v, np.array([n]))


def test_ring_comparison_rejects_a_wrong_value_row():
    """Keys and positions right; one slot holds another token's value row."""
    n = 9
    k, v = data(n)
    bad = Ring(k, v, n)
    s = (n - 1) % W
    bad.v[0, :, s] = torch.from_numpy(v[0, :, n - 2].view(np.int16)).view(torch.bfloat16)
    with pytest.raises(AssertionError):
        check_ring_rows(bad, k, v, np.array([n]))


class DitherCache:
    """A Tier B ring cache (B = 1, H = 1) as CPU tensors, filled from the
    oracle's own quantization: the layout check_dither_store reads."""

    def __init__(self, n=16 * 4 + 6, w=48, seed=6, req=21, layer=2):
        rng = np.random.default_rng(seed)
        self.W, self.B, self.layer, self.layout = w, 1, layer, "ring"
        self.n = n
        self.kbits, self.k64 = _bf16_rows(rng, n, 128)
        self.vbits, self.v64 = _bf16_rows(rng, n, 128)
        self.request_id = torch.tensor([req], dtype=torch.int64)
        nb = n // 16
        k = np.zeros((1, 1, w, 128), dtype=np.int8)
        v = np.zeros_like(k)
        ks = np.zeros((1, 1, w // 16), dtype=np.float32)
        vs = np.zeros_like(ks)
        pos = np.full((1, w), -1, dtype=np.int32)
        for kb in range(max(0, nb - w // 16), nb):
            rows = np.arange(16 * kb, 16 * kb + 16)
            u = odither.dither(req, layer, 0, rows, 128)
            sk, ck = odither.quantize_block(self.k64[rows], u)
            sv, cv = odither.quantize_block(self.v64[rows], u)
            s0 = (16 * kb) % w
            k[0, 0, s0:s0 + 16], v[0, 0, s0:s0 + 16] = ck, cv
            ks[0, 0, s0 // 16], vs[0, 0, s0 // 16] = sk, sv
            pos[0, s0:s0 + 16] = rows
        ksg = np.zeros((1, 1, 16, 128), dtype=np.uint16)
        vsg = np.zeros_like(ksg)
        for p in range(16 * nb, n):
            ksg[0, 0, p % 16], vsg[0, 0, p % 16] = self.kbits[p], self.vbits[p]
        self.k, self.v = torch.from_numpy(k), torch.from_numpy(v)
        self.k_scale, self.v_scale = torch.from_numpy(ks), torch.from_numpy(vs)
        self.pos = torch.from_numpy(pos)
        self.k_stage = torch.from_numpy(ksg.view(np.int16)).view(torch.bfloat16)
        self.v_stage = torch.from_numpy(vsg.view(np.int16)).view(torch.bfloat16)

    def check(self):
        check_dither_store(self, 0, 0, self.k64, self.v64, self.n)


def test_dither_store_comparison_accepts_the_oracle_state():
    DitherCache().check()


@pytest.mark.parametrize("field", ["k_codes", "v_codes", "k_scale", "v_scale", "pos", "k_stage", "v_stage"])
def test_dither_store_comparison_rejects_each_field(field):
    c = DitherCache()
    slot = 20
    if field == "k_codes":
        c.k[0, 0, slot, 3] += 1 if c.k[0, 0, slot, 3] < 127 else -1
    elif field == "v_codes":
        c.v[0, 0, slot, 3] += 1 if c.v[0, 0, slot, 3] < 127 else -1
    elif field == "k_scale":
        c.k_scale[0, 0, slot // 16] *= 1.5
    elif field == "v_scale":
        c.v_scale[0, 0, slot // 16] *= 1.5
    elif field == "pos":
        c.pos[0, slot] += c.W
    elif field == "k_stage":
        c.k_stage.view(torch.int16)[0, 0, (c.n - 1) % 16, 9] ^= 1
    elif field == "v_stage":
        c.v_stage.view(torch.int16)[0, 0, (c.n - 1) % 16, 9] ^= 1
    with pytest.raises(AssertionError):
        c.check()
