"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same split policy, same entry points).  Outputs are compared
with the float64 oracle on every (b, h) pair where the oracle is fast enough,
otherwise on seeded samples of pairs; ring state is compared bit-exactly on
sampled sequences and checked everywhere with swa_validate.
"""

import numpy as np
import pytest
import torch

import workloads
from workloads import gen
from oracle import attention, decoder
from tests.gpu_util import (assert_close, check_dither_decode, check_dither_store, check_int8_decode,
                            check_int8_store, f64, host_bits, request_ids, require_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def prefill(swa, cache, k_all, v_all, n, chunk):
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        swa.kv_append(cache, k_all[:, :, c0:c1].contiguous(), v_all[:, :, c0:c1].contiguous())


def test_full_cache_ragged_4096():
    """B=8, H=32, D=128, capacity 4096, lengths U{1024..4096}: all 256 pairs,
    after the per-sequence prefill and after one fused step (decode_step, the
    benchmark's call; a sequence at length 4096 wraps)."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.FULL_RAGGED
    lens = gen.ragged_lengths(wl)
    say("ragged lengths", lens.tolist())
    dev = torch.device("cuda")
    k_all = gen.tokens(wl, "k", wl.W, device=dev)
    v_all = gen.tokens(wl, "v", wl.W, device=dev)
    cache = swa.KVCache("bf16", wl.B, wl.H, wl.D, wl.W)
    for b, n in enumerate(lens):
        swa.kv_append(cache.seq_view(b), k_all[b:b + 1, :, :n].contiguous(), v_all[b:b + 1, :, :n].contiguous())
    q = gen.query(wl, 0, device=dev)
    out = swa.decode_attn(cache, q).cpu().numpy()
    assert swa.validate(cache) == 0
    assert host_bits(cache.next_position).tolist() == lens.tolist()
    q64 = f64(q)
    worst = 0.0
    for b, n in enumerate(lens):
        k64, v64 = f64(k_all[b, :, :n]), f64(v_all[b, :, :n])
        for h in range(wl.H):
            ref = attention.masked_attention(q64[b, h], np.arange(n), k64[h], v64[h], n - 1, wl.W)
            worst = max(worst, assert_close(out[b, h], ref, f"ragged b={b} h={h}"))
    # one fused step (the benchmark's call): every sequence appends a token at its own position
    g = torch.Generator(device="cuda").manual_seed(21)
    kn = torch.randn((wl.B, wl.H, 1, wl.D), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((wl.B, wl.H, 1, wl.D), generator=g, device=dev).to(torch.bfloat16)
    q2 = gen.query(wl, 1, device=dev)
    out2 = swa.decode_step(cache, kn, vn, q2).cpu().numpy()
    assert host_bits(cache.next_position).tolist() == (lens + 1).tolist()
    assert swa.validate(cache) == 0
    q64 = f64(q2)
    for b, n in enumerate(lens):
        k64 = np.concatenate([f64(k_all[b, :, :n]), f64(kn[b])], axis=1)
        v64 = np.concatenate([f64(v_all[b, :, :n]), f64(vn[b])], axis=1)
        for h in range(wl.H):
            ref = attention.masked_attention(q64[b, h], np.arange(n + 1), k64[h], v64[h], n, wl.W)
            worst = max(worst, assert_close(out2[b, h], ref, f"ragged step b={b} h={h}"))
    say(f"ragged max abs err {worst:.2e}")


def test_ring_w4096_positions_8192_to_8447():
    """B=16, H=32, W=4096: prefill 0..8191 in two chunks, then 256 append+attend
    steps, alternately the fused decode_step (the benchmark's call) and
    kv_append + decode_attn; every step checks 4 sampled pairs and the
    position invariant; ring
    bits of sampled sequences are compared at the first, a middle and the
    last step.  The sampled pairs rotate over a fixed seeded set of 8."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.RING
    dev = torch.device("cuda")
    total = wl.prefill + wl.steps
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    cache = swa.KVCache("bf16", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(3)
    pairs = [(int(rng.integers(wl.B)), int(rng.integers(wl.H))) for _ in range(8)]
    hist64 = {bh: (f64(k_all[bh[0], bh[1]]), f64(v_all[bh[0], bh[1]])) for bh in pairs}
    worst = 0.0
    for i in range(wl.steps):
        p = wl.prefill + i
        q = gen.query(wl, p, device=dev)
        kn, vn = k_all[:, :, p:p + 1].contiguous(), v_all[:, :, p:p + 1].contiguous()
        if i % 2 == 0:  # the benchmark's call: the fused step
            out = swa.decode_step(cache, kn, vn, q)
        else:
            swa.kv_append(cache, kn, vn)
            out = swa.decode_attn(cache, q)
        assert swa.validate(cache) == 0, f"step {p}"
        outh = out.cpu().numpy()
        qh = f64(q)
        for j in range(4):
            b, h = pairs[(4 * i + j) % len(pairs)]
            k64, v64 = hist64[(b, h)]
            ref = attention.masked_attention(qh[b, h], np.arange(p + 1), k64[:p + 1], v64[:p + 1], p, wl.W)
            worst = max(worst, assert_close(outh[b, h], ref, f"ring step {p} b={b} h={h}"))
        if i in (0, wl.steps // 2, wl.steps - 1):
            b = int(rng.integers(wl.B))
            exp = decoder.expected_ring(np.arange(p + 1), wl.W)
            np.testing.assert_array_equal(host_bits(cache.pos[b]), exp)
            kb = host_bits(cache.k[b])
            np.testing.assert_array_equal(kb, host_bits(k_all[b][:, torch.as_tensor(exp, device=dev)]))
    say(f"ring max abs err {worst:.2e}")


def test_long_context_131072_spiked():
    """B=4, H=8, W=131072 with 1% of keys x8: all 32 pairs, after prefill and
    after one fused step (decode_step, the benchmark's call) that wraps the
    ring."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.LONG
    dev = torch.device("cuda")
    k_all = gen.tokens(wl, "k", wl.W, device=dev)
    v_all = gen.tokens(wl, "v", wl.W, device=dev)
    cache = swa.KVCache("bf16", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.W, 32768)
    q = gen.query(wl, wl.W - 1, device=dev)
    out = swa.decode_attn(cache, q).cpu().numpy()
    assert swa.validate(cache) == 0
    q64 = f64(q)
    worst = 0.0
    for b in range(wl.B):
        for h in range(wl.H):
            k64, v64 = f64(k_all[b, h]), f64(v_all[b, h])
            ref = attention.masked_attention(q64[b, h], np.arange(wl.W), k64, v64, wl.W - 1, wl.W)
            worst = max(worst, assert_close(out[b, h], ref, f"long b={b} h={h}"))
    # one fused step (the benchmark's call): position 131072 overwrites slot 0
    g = torch.Generator(device="cuda").manual_seed(22)
    kn = torch.randn((wl.B, wl.H, 1, wl.D), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((wl.B, wl.H, 1, wl.D), generator=g, device=dev).to(torch.bfloat16)
    q2 = gen.query(wl, wl.W, device=dev)
    out2 = swa.decode_step(cache, kn, vn, q2).cpu().numpy()
    assert swa.validate(cache) == 0
    q64 = f64(q2)
    for b in range(wl.B):
        for h in range(wl.H):
            k64 = np.concatenate([f64(k_all[b, h]), f64(kn[b, h])])
            v64 = np.concatenate([f64(v_all[b, h]), f64(vn[b, h])])
            ref = attention.masked_attention(q64[b, h], np.arange(wl.W + 1), k64, v64, wl.W, wl.W)
            worst = max(worst, assert_close(out2[b, h], ref, f"long step b={b} h={h}"))
    say(f"long-context max abs err {worst:.2e}")


def test_bf16_ctx32768_sampled():
    """B=16, H=32, W=32768 bf16 (rotary keys): 8 sampled pairs after prefill
    and 2 after each of 3 fused steps (decode_step, the benchmark's call)."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.BF16_32K
    dev = torch.device("cuda")
    total = wl.prefill + 3
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    cache = swa.KVCache("bf16", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(5)
    n = wl.prefill
    for extra in range(4):
        if extra:  # the benchmark's call: the fused step
            q = gen.query(wl, n, device=dev)
            out = swa.decode_step(cache, k_all[:, :, n:n + 1].contiguous(), v_all[:, :, n:n + 1].contiguous(),
                                  q).cpu().numpy()
            n += 1
        else:
            q = gen.query(wl, n - 1, device=dev)
            out = swa.decode_attn(cache, q).cpu().numpy()
        qh = f64(q)
        for _ in range(2 if extra else 8):
            b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
            k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
            ref = attention.masked_attention(qh[b, h], np.arange(n), k64, v64, n - 1, wl.W)
            assert_close(out[b, h], ref, f"bf16-32k n={n} b={b} h={h}")
    assert swa.validate(cache) == 0


def test_int8_witness_ctx32768():
    """B=16, H=32, W=32768 INT8 with rotary keys: after the 32768-token
    prefill, 3 sampled pairs get the full store check (codes, scales bits,
    witness >= exact norms) and the per-token bound check; then 20 steps at
    positions 32768..32787 (crossing the block boundary at 32784), alternately
    the fused decode_step_int8 (the benchmark's call) and kv_append + the
    decode, check one pair each."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.INT8_32K
    dev = torch.device("cuda")
    total = wl.prefill + wl.steps
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    cache = swa.KVCache("int8", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(8)
    n = wl.prefill
    q = gen.query(wl, n - 1, device=dev)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q, want_c_all=True)
    assert swa.validate(cache) == 0
    out, cmax, c_all, qh = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy(), f64(q)
    for _ in range(3):
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
        say("int8 32k store check", b, h)
        check_int8_store(cache, b, h, k64, v64, n)
        check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, qh[b, h], k64, v64, n, wl.W, "32k")
    for i in range(wl.steps):
        kn, vn = k_all[:, :, n:n + 1].contiguous(), v_all[:, :, n:n + 1].contiguous()
        q = gen.query(wl, n, device=dev)
        if i % 2 == 1:  # the benchmark's call: the fused step (no c_all)
            out, cmax, _, _ = swa.decode_step_int8(cache, kn, vn, q)
            c_all = None
        else:
            swa.kv_append(cache, kn, vn)
            out, cmax, c_all = swa.decode_attn_int8_witness(cache, q, want_c_all=True)
        n += 1
        assert swa.validate(cache) == 0
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
        check_int8_decode(out[b, h].cpu().numpy(), float(cmax[b, h]),
                          None if c_all is None else c_all[b, h].cpu().numpy(), b, h, f64(q[b, h]), k64, v64, n,
                          wl.W, f"32k step n={n}")
    say("int8 32k steps ok, last n", n)


def test_int8_dither_ctx32768():
    """The INT8 32k inputs stored with subtractive dither (request ids 0..15,
    layer 0), decoded with delta = 1e-6 as the benchmark does: after the
    prefill, 2 sampled pairs get the full store check (codes and scales bit
    for bit against the oracle's own Philox stream) and the decode check;
    then 20 steps at positions 32768..32787, alternately the fused
    decode_step_int8 (the benchmark's call) and kv_append + the decode, with
    the decode of one pair checked at six of them, including both sides of
    the block commit at 32784."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.INT8_DITHER_32K
    delta = 1e-6
    dev = torch.device("cuda")
    total = wl.prefill + wl.steps
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    cache = swa.KVCache("int8_dither", wl.B, wl.H, wl.D, wl.W)
    reqs = request_ids(cache)
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(9)
    n = wl.prefill
    q = gen.query(wl, n - 1, device=dev)
    out, cert, tv, gate = swa.decode_attn_int8_dither(cache, q, delta=delta)
    assert swa.validate(cache) == 0
    out, cert, tv, gate, qh = out.cpu().numpy(), cert.cpu().numpy(), tv.cpu().numpy(), gate.cpu().numpy(), f64(q)
    for _ in range(2):
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
        say("dither 32k store check", b, h)
        check_dither_store(cache, b, h, k64, v64, n)
        check_dither_decode(out[b, h], cert[b, h], b, h, qh[b, h], k64, v64, n, wl.W, reqs[b], cache.layer, delta,
                            tv[b, h], gate[b, h], what="32k")
    for i in range(wl.steps):
        kn, vn = k_all[:, :, n:n + 1].contiguous(), v_all[:, :, n:n + 1].contiguous()
        q = gen.query(wl, n, device=dev)
        if i % 2 == 1:  # the benchmark's call: the fused step
            out, cert, tv, gate = swa.decode_step_int8(cache, kn, vn, q, delta=delta, want_tv=True)
        else:
            swa.kv_append(cache, kn, vn)
            out, cert, tv, gate = swa.decode_attn_int8_dither(cache, q, delta=delta)
        n += 1
        assert swa.validate(cache) == 0
        if i not in (0, 7, 14, 15, 16, 19):
            continue
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
        check_dither_decode(out[b, h].cpu().numpy(), float(cert[b, h]), b, h, f64(q[b, h]), k64, v64, n, wl.W, reqs[b],
                            cache.layer, delta, float(tv[b, h]), int(gate[b, h]), what=f"32k step n={n}")
    say("dither 32k steps ok, last n", n)


def test_long_context_shard_16384_spiked():
    """One GPU's share of the 131072 context split 8 ways: B=4, H=8,
    W=16384 with 1% of keys x8, all 32 pairs, through decode_step (the
    benchmark's call; several splits per pair, so append + decode + merge)."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.LONG_CTX_SHARD
    dev = torch.device("cuda")
    n = wl.prefill + 1
    k_all = gen.tokens(wl, "k", n, device=dev)
    v_all = gen.tokens(wl, "v", n, device=dev)
    cache = swa.KVCache("bf16", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.prefill, 8192)
    q = gen.query(wl, n - 1, device=dev)
    out = swa.decode_step(cache, k_all[:, :, n - 1:n].contiguous(), v_all[:, :, n - 1:n].contiguous(), q)
    out = out.cpu().numpy()
    assert swa.validate(cache) == 0
    assert host_bits(cache.next_position).tolist() == [n] * wl.B
    q64 = f64(q)
    worst = 0.0
    for b in range(wl.B):
        for h in range(wl.H):
            k64, v64 = f64(k_all[b, h]), f64(v_all[b, h])
            ref = attention.masked_attention(q64[b, h], np.arange(n), k64, v64, n - 1, wl.W)
            worst = max(worst, assert_close(out[b, h], ref, f"ctx shard b={b} h={h}"))
    say(f"context-shard max abs err {worst:.2e}")


def test_int8_head_shard_ctx32768():
    """One GPU's 4 of the 32 heads of the INT8 32k workload: B=16, H=4,
    W=32768.  After prefill, 3 sampled pairs get the store and per-token bound
    checks; then 20 decode_step_int8 calls (the benchmark's call; several
    splits per pair, so the separate launches) at positions 32768..32787 check
    one pair each, with the cache state validated every step."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.INT8_HEAD_SHARD
    dev = torch.device("cuda")
    total = wl.prefill + wl.steps
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    cache = swa.KVCache("int8", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(9)
    n = wl.prefill
    q = gen.query(wl, n - 1, device=dev)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q, want_c_all=True)
    out, cmax, c_all, qh = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy(), f64(q)
    for _ in range(3):
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
        say("int8 head shard store check", b, h)
        check_int8_store(cache, b, h, k64, v64, n)
        check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, qh[b, h], k64, v64, n, wl.W, "head shard")
    for i in range(wl.steps):
        q = gen.query(wl, n, device=dev)
        out, cmax, _, _ = swa.decode_step_int8(cache, k_all[:, :, n:n + 1].contiguous(),
                                               v_all[:, :, n:n + 1].contiguous(), q)
        n += 1
        assert swa.validate(cache) == 0
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
        check_int8_decode(out[b, h].cpu().numpy(), float(cmax[b, h]), None, b, h, f64(q[b, h]), k64, v64, n,
                          wl.W, f"head shard step n={n}")
    say("int8 head shard steps ok, last n", n)


def test_int8_witness_ctx32768_paged():
    """The INT8 32k workload in 16-token pages (shuffled table over the pool):
    after the prefill, 2 sampled pairs get the store check (read back through
    the table) and the per-token bound check; then 18 steps up to and past
    the block commit at 32784, alternately the fused decode_step_int8 (the
    benchmark's call) and kv_append + the decode, check one pair each."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.INT8_32K_PAGED
    dev = torch.device("cuda")
    total = wl.prefill + 18
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    cache = swa.KVCache("int8", wl.B, wl.H, wl.D, wl.W, layout="paged")
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(18)
    n = wl.prefill
    q = gen.query(wl, n - 1, device=dev)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q, want_c_all=True)
    assert swa.validate(cache) == 0
    out, cmax, c_all, qh = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy(), f64(q)
    for _ in range(2):
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
        say("int8 32k paged store check", b, h)
        check_int8_store(cache, b, h, k64, v64, n)
        check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, qh[b, h], k64, v64, n, wl.W, "32k paged")
    for i in range(18):
        kn, vn = k_all[:, :, n:n + 1].contiguous(), v_all[:, :, n:n + 1].contiguous()
        q = gen.query(wl, n, device=dev)
        if i % 2 == 1:
            out, cmax, _, _ = swa.decode_step_int8(cache, kn, vn, q)
        else:
            swa.kv_append(cache, kn, vn)
            out, cmax, _ = swa.decode_attn_int8_witness(cache, q)
        n += 1
        assert swa.validate(cache) == 0
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
        check_int8_decode(out[b, h].cpu().numpy(), float(cmax[b, h]), None, b, h, f64(q[b, h]), k64, v64, n, wl.W,
                          f"32k paged step n={n}")
    b = int(rng.integers(wl.B))
    check_int8_store(cache, b, 0, f64(k_all[b, 0, :n]), f64(v_all[b, 0, :n]), n)
    say("int8 32k paged steps ok, last n", n)


def test_bf16_ctx32768_paged_sampled():
    """The bf16 32k workload in 16-token pages: 6 sampled pairs after the
    prefill, then 3 fused steps (decode_step, the benchmark's call) with 2
    sampled pairs each; ring rows of one sequence read back through the
    table bit for bit."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.BF16_32K_PAGED
    dev = torch.device("cuda")
    total = wl.prefill + 3
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    cache = swa.KVCache("bf16", wl.B, wl.H, wl.D, wl.W, layout="paged")
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(19)
    n = wl.prefill
    for extra in range(4):
        if extra:
            q = gen.query(wl, n, device=dev)
            out = swa.decode_step(cache, k_all[:, :, n:n + 1].contiguous(), v_all[:, :, n:n + 1].contiguous(),
                                  q).cpu().numpy()
            n += 1
        else:
            q = gen.query(wl, n - 1, device=dev)
            out = swa.decode_attn(cache, q).cpu().numpy()
        assert swa.validate(cache) == 0
        qh = f64(q)
        for _ in range(2 if extra else 6):
            b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
            k64, v64 = f64(k_all[b, h, :n]), f64(v_all[b, h, :n])
            ref = attention.masked_attention(qh[b, h], np.arange(n), k64, v64, n - 1, wl.W)
            assert_close(out[b, h], ref, f"bf16-32k paged n={n} b={b} h={h}")
    from tests.gpu_util import RingView
    view = RingView(cache)
    b = int(rng.integers(wl.B))
    exp = decoder.expected_ring(np.arange(n), wl.W)
    np.testing.assert_array_equal(host_bits(view.pos[b]), exp)
    np.testing.assert_array_equal(host_bits(view.k[b]), host_bits(k_all[b][:, torch.as_tensor(exp, device=dev)]))
