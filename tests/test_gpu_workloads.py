"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same split policy, same entry points).  Every (b, h) pair of
every workload is compared with the float64 oracle at least once: the
cheap ones in the test process, the 32k ones (about 1.4 s of oracle per INT8
pair) in a pool of host processes (tests/oracle_pool.py).  Ring state is
compared bit-exactly and checked everywhere with swa_validate.
"""

import numpy as np
import pytest
import torch

import workloads
from workloads import gen
from oracle import attention, bits, decoder
from tests import oracle_pool
from tests.gpu_util import (RingView, assert_close, check_dither_decode, check_dither_store, check_int8_decode,
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


def rows_all_pairs(kb, vb, qb, n, W, out, label):
    """Every (b, h) of a row cache after n tokens per sequence: the output vs
    the oracle's masked attention, in the host pool.  kb, vb [B, H, >=n, D]
    and qb [B, H, D] are host bits; out [B, H, D] the GPU's output."""
    B, H = out.shape[:2]
    tasks = [(kb[b, h, :n], vb[b, h, :n], qb[b, h], n, W, out[b, h], f"{label} b={b} h={h}")
             for b in range(B) for h in range(H)]
    return oracle_pool.run(oracle_pool.rows_task, tasks, label)


def host_store(view):
    """Host copies of an INT8 cache's storage in ring order (a ring cache, or
    a RingView of a paged one), as check_int8_store_arrays takes them."""
    return (host_bits(view.k), host_bits(view.v), host_bits(view.k_scale), host_bits(view.v_scale),
            host_bits(view.witness).view(np.float16).astype(np.float64), host_bits(view.pos),
            host_bits(view.k_stage), host_bits(view.v_stage))


def int8_all_pairs(kb, vb, qb, n, W, out, cmax, c_all, label, store=None):
    """Every (b, h) of an INT8 cache after n tokens per sequence: output,
    cmax and (when given) every per-token c_t vs the oracle, and (when the
    host_store copies are given) the whole store of the pair, in the host
    pool."""
    B, H = out.shape[:2]

    def pair_store(b, h):
        kc, vc, ks, vs, wit, pos, ksg, vsg = store
        return kc[b, h], vc[b, h], ks[b, h], vs[b, h], wit[b, h], pos[b], ksg[b, h], vsg[b, h]

    tasks = [(kb[b, h, :n], vb[b, h, :n], qb[b, h], n, W, b, h, out[b, h], float(cmax[b, h]),
              None if c_all is None else c_all[b, h], None if store is None else pair_store(b, h), label)
             for b in range(B) for h in range(H)]
    return oracle_pool.run(oracle_pool.int8_task, tasks, label)


def dither_all_pairs(kb, vb, qb, n, W, out, cert, tv, gate, reqs, layer, delta, label):
    """Every (b, h) of a Tier B cache after n tokens per sequence: output,
    certificate, tv and gate vs the oracle, in the host pool."""
    B, H = out.shape[:2]
    tasks = [(kb[b, h, :n], vb[b, h, :n], qb[b, h], n, W, b, h, out[b, h], float(cert[b, h]), float(tv[b, h]),
              int(gate[b, h]), reqs[b], layer, delta, label) for b in range(B) for h in range(H)]
    return oracle_pool.run(oracle_pool.dither_task, tasks, label)


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


@pytest.mark.timeout(600)
def test_ring_w4096_positions_8192_to_8447():
    """B=16, H=32, W=4096: prefill 0..8191 in two chunks, then 256 append+attend
    steps, alternately the fused decode_step (the benchmark's call) and
    kv_append + decode_attn.  At the first, a middle and the last step all
    512 pairs are compared with the oracle, and the whole ring (positions, K
    and V bits of every sequence) with what it must hold; every other step
    compares 4 pairs, walking a seeded permutation of all 512 pairs, and
    checks the position invariant."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.RING
    dev = torch.device("cuda")
    total = wl.prefill + wl.steps
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    kb, vb = host_bits(k_all), host_bits(v_all)
    cache = swa.KVCache("bf16", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(3)
    order = [divmod(int(x), wl.H) for x in rng.permutation(wl.B * wl.H)]
    full = (0, wl.steps // 2, wl.steps - 1)
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
        pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)] if i in full else \
            [order[(4 * i + j) % len(order)] for j in range(4)]
        for b, h in pairs:
            k64, v64 = bits.to_f64(kb[b, h, :p + 1]), bits.to_f64(vb[b, h, :p + 1])
            ref = attention.masked_attention(qh[b, h], np.arange(p + 1), k64, v64, p, wl.W)
            worst = max(worst, assert_close(outh[b, h], ref, f"ring step {p} b={b} h={h}"))
        if i in full:
            exp = decoder.expected_ring(np.arange(p + 1), wl.W)
            ex = torch.as_tensor(exp, device=dev)
            assert (exp >= 0).all()
            for b in range(wl.B):
                np.testing.assert_array_equal(host_bits(cache.pos[b]), exp)
            assert torch.equal(cache.k, k_all[:, :, ex]), f"ring K bits at step {p}"
            assert torch.equal(cache.v, v_all[:, :, ex]), f"ring V bits at step {p}"
            say(f"ring step {p}: all pairs and the whole ring checked, worst {worst:.2e}")
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


@pytest.mark.timeout(600)
def test_bf16_ctx32768_all_pairs():
    """B=16, H=32, W=32768 bf16 (rotary keys): all 512 pairs after prefill
    and after the third of 3 fused steps (decode_step, the benchmark's call),
    2 sampled pairs after each of the first two."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.BF16_32K
    dev = torch.device("cuda")
    total = wl.prefill + 3
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    kb, vb = host_bits(k_all), host_bits(v_all)
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
        assert swa.validate(cache) == 0
        if extra in (0, 3):
            rows_all_pairs(kb, vb, host_bits(q), n, wl.W, out, f"bf16-32k n={n}")
            continue
        qh = f64(q)
        for _ in range(2):
            b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
            ref = attention.masked_attention(qh[b, h], np.arange(n), bits.to_f64(kb[b, h, :n]),
                                             bits.to_f64(vb[b, h, :n]), n - 1, wl.W)
            assert_close(out[b, h], ref, f"bf16-32k n={n} b={b} h={h}")


@pytest.mark.timeout(900)
def test_int8_witness_ctx32768():
    """B=16, H=32, W=32768 INT8 with rotary keys.  After the 32768-token
    prefill, all 512 pairs get the full store check (codes and scales bit for
    bit, witness >= the exact band norms) and the decode check with every
    per-token bound c_t.  Then 20 steps at positions 32768..32787,
    alternately the fused decode_step_int8 (the benchmark's call) and
    kv_append + the decode, check one pair each, except the fused step that
    commits block 2048 (position 32783, n = 32784 after it): there all 512
    pairs are checked, and 8 sampled pairs get the store check."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.INT8_32K
    dev = torch.device("cuda")
    total = wl.prefill + wl.steps
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    kb, vb = host_bits(k_all), host_bits(v_all)
    cache = swa.KVCache("int8", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(8)
    n = wl.prefill
    q = gen.query(wl, n - 1, device=dev)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q, want_c_all=True)
    assert swa.validate(cache) == 0
    worst = int8_all_pairs(kb, vb, host_bits(q), n, wl.W, out.cpu().numpy(), cmax.cpu().numpy(),
                           c_all.cpu().numpy(), "int8 32k prefill", store=host_store(cache))
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
        if n == 32784:  # the fused step that committed block 2048
            assert i % 2 == 1
            worst = max(worst, int8_all_pairs(kb, vb, host_bits(q), n, wl.W, out.cpu().numpy(),
                                              cmax.cpu().numpy(), None, "int8 32k commit step"))
            for _ in range(8):
                b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
                check_int8_store(cache, b, h, bits.to_f64(kb[b, h, :n]), bits.to_f64(vb[b, h, :n]), n)
            continue
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        check_int8_decode(out[b, h].cpu().numpy(), float(cmax[b, h]),
                          None if c_all is None else c_all[b, h].cpu().numpy(), b, h, f64(q[b, h]),
                          bits.to_f64(kb[b, h, :n]), bits.to_f64(vb[b, h, :n]), n, wl.W, f"32k step n={n}")
    say(f"int8 32k steps ok, last n {n}, worst abs err {worst:.2e}")


@pytest.mark.timeout(600)
def test_int8_dither_ctx32768():
    """The INT8 32k inputs stored with subtractive dither (request ids 0..15,
    layer 0), decoded with delta = 1e-6 as the benchmark does: after the
    prefill, 2 sampled pairs get the full store check (codes and scales bit
    for bit against the oracle's own Philox stream) and the decode check;
    then 20 steps at positions 32768..32787, alternately the fused
    decode_step_int8 (the benchmark's call) and kv_append + the decode.  At
    the fused step that commits block 2048 (n = 32784 after it) all 512 pairs
    are checked; five other steps check one pair each."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.INT8_DITHER_32K
    delta = 1e-6
    dev = torch.device("cuda")
    total = wl.prefill + wl.steps
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    kb, vb = host_bits(k_all), host_bits(v_all)
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
        k64, v64 = bits.to_f64(kb[b, h, :n]), bits.to_f64(vb[b, h, :n])
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
        if n == 32784:  # the fused step that committed block 2048
            assert i % 2 == 1
            dither_all_pairs(kb, vb, host_bits(q), n, wl.W, out.cpu().numpy(), cert.cpu().numpy(),
                             tv.cpu().numpy(), gate.cpu().numpy(), reqs, cache.layer, delta, "dither 32k commit step")
            continue
        if i not in (0, 7, 14, 16, 19):
            continue
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        check_dither_decode(out[b, h].cpu().numpy(), float(cert[b, h]), b, h, f64(q[b, h]),
                            bits.to_f64(kb[b, h, :n]), bits.to_f64(vb[b, h, :n]), n, wl.W, reqs[b], cache.layer, delta,
                            float(tv[b, h]), int(gate[b, h]), what=f"32k step n={n}")
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


@pytest.mark.timeout(600)
def test_int8_head_shard_ctx32768():
    """One GPU's 4 of the 32 heads of the INT8 32k workload: B=16, H=4,
    W=32768.  After prefill, all 64 pairs get the store check and the
    per-token bound check; then 20 decode_step_int8 calls (the benchmark's
    call; several splits per pair, so the separate launches) at positions
    32768..32787 check one pair each, with the cache state validated every
    step, and all 64 pairs after the last."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.INT8_HEAD_SHARD
    dev = torch.device("cuda")
    total = wl.prefill + wl.steps
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    kb, vb = host_bits(k_all), host_bits(v_all)
    cache = swa.KVCache("int8", wl.B, wl.H, wl.D, wl.W)
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(9)
    n = wl.prefill
    q = gen.query(wl, n - 1, device=dev)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q, want_c_all=True)
    int8_all_pairs(kb, vb, host_bits(q), n, wl.W, out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy(),
                   "int8 head shard prefill", store=host_store(cache))
    for i in range(wl.steps):
        q = gen.query(wl, n, device=dev)
        out, cmax, _, _ = swa.decode_step_int8(cache, k_all[:, :, n:n + 1].contiguous(),
                                               v_all[:, :, n:n + 1].contiguous(), q)
        n += 1
        assert swa.validate(cache) == 0
        if i == wl.steps - 1:
            int8_all_pairs(kb, vb, host_bits(q), n, wl.W, out.cpu().numpy(), cmax.cpu().numpy(), None,
                           "int8 head shard last step")
            break
        b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
        check_int8_decode(out[b, h].cpu().numpy(), float(cmax[b, h]), None, b, h, f64(q[b, h]),
                          bits.to_f64(kb[b, h, :n]), bits.to_f64(vb[b, h, :n]), n, wl.W, f"head shard step n={n}")
    say("int8 head shard steps ok, last n", n)


@pytest.mark.timeout(900)
def test_int8_witness_ctx32768_paged():
    """The INT8 32k workload in 16-token pages (shuffled table over the pool):
    after the prefill, all 512 pairs get the store check (read back through
    the table) and the decode check with every per-token bound; then 18
    steps up to and past the block commit at 32784, alternately the fused
    decode_step_int8 (the benchmark's call) and kv_append + the decode, check
    one pair each."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.INT8_32K_PAGED
    dev = torch.device("cuda")
    total = wl.prefill + 18
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    kb, vb = host_bits(k_all), host_bits(v_all)
    cache = swa.KVCache("int8", wl.B, wl.H, wl.D, wl.W, layout="paged")
    prefill(swa, cache, k_all, v_all, wl.prefill, wl.prefill_chunk)
    rng = np.random.default_rng(18)
    n = wl.prefill
    q = gen.query(wl, n - 1, device=dev)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q, want_c_all=True)
    assert swa.validate(cache) == 0
    int8_all_pairs(kb, vb, host_bits(q), n, wl.W, out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy(),
                   "int8 32k paged prefill", store=host_store(RingView(cache)))
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
        check_int8_decode(out[b, h].cpu().numpy(), float(cmax[b, h]), None, b, h, f64(q[b, h]),
                          bits.to_f64(kb[b, h, :n]), bits.to_f64(vb[b, h, :n]), n, wl.W, f"32k paged step n={n}")
    b = int(rng.integers(wl.B))
    check_int8_store(cache, b, 0, bits.to_f64(kb[b, 0, :n]), bits.to_f64(vb[b, 0, :n]), n)
    say("int8 32k paged steps ok, last n", n)


@pytest.mark.timeout(600)
def test_bf16_ctx32768_paged_all_pairs():
    """The bf16 32k workload in 16-token pages: all 512 pairs after the
    prefill and after the last of 3 fused steps (decode_step, the benchmark's
    call), 2 sampled pairs after the others; ring rows of one sequence read
    back through the table bit for bit."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.BF16_32K_PAGED
    dev = torch.device("cuda")
    total = wl.prefill + 3
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    kb, vb = host_bits(k_all), host_bits(v_all)
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
        if extra in (0, 3):
            rows_all_pairs(kb, vb, host_bits(q), n, wl.W, out, f"bf16-32k paged n={n}")
            continue
        qh = f64(q)
        for _ in range(2):
            b, h = int(rng.integers(wl.B)), int(rng.integers(wl.H))
            ref = attention.masked_attention(qh[b, h], np.arange(n), bits.to_f64(kb[b, h, :n]),
                                             bits.to_f64(vb[b, h, :n]), n - 1, wl.W)
            assert_close(out[b, h], ref, f"bf16-32k paged n={n} b={b} h={h}")
    view = RingView(cache)
    b = int(rng.integers(wl.B))
    exp = decoder.expected_ring(np.arange(n), wl.W)
    np.testing.assert_array_equal(host_bits(view.pos[b]), exp)
    np.testing.assert_array_equal(host_bits(view.k[b]), host_bits(k_all[b][:, torch.as_tensor(exp, device=dev)]))
