"""Helpers for the GPU parity tests: device checks, host copies of device
tensors, and comparisons of the HIP results with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import bits, decoder, dither as odither, int8 as oint8

TOL = 2e-3  # max abs error of outputs vs the float64 oracle on the same inputs


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


def check_int8_store(cache, b: int, h: int, k64: np.ndarray, v64: np.ndarray, n: int):
    """INT8 cache of (b, h): codes, scales, slot positions bit-exact vs the
    oracle; stored witness never below the exact band norm and within one
    fp16 step above it; staging rows equal the input bits."""
    if getattr(cache, "layout", "ring") == "paged":
        cache = RingView(cache)
    st = decoder.expected_int8_store(k64, v64, n, cache.W)
    kc = host_bits(cache.k[b, h]); vc = host_bits(cache.v[b, h])
    ks = host_bits(cache.k_scale[b, h]); vs = host_bits(cache.v_scale[b, h])
    wit = host_bits(cache.witness[b, h]).view(np.float16).astype(np.float64)
    pos = host_bits(cache.pos[b])
    np.testing.assert_array_equal(pos, st["slot_pos"])
    live = np.nonzero(st["slot_pos"] >= 0)[0]
    np.testing.assert_array_equal(kc[live], st["k_codes"][live])
    np.testing.assert_array_equal(vc[live], st["v_codes"][live])
    lb = np.unique(live // 16)
    np.testing.assert_array_equal(ks[lb], st["k_scale"][lb])
    np.testing.assert_array_equal(vs[lb], st["v_scale"][lb])
    we, wg = st["witness"][live], wit[live]
    assert np.all(wg >= we), "stored witness below the exact band norm"
    assert np.all(wg <= we * (1 + 2.0 ** -9) + 2.0 ** -24), "stored witness not tight"
    ksg = host_bits(cache.k_stage[b, h]); vsg = host_bits(cache.v_stage[b, h])
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
