"""GPU parity of the row (bf16/fp32) ring cache through the C ABI.

Ring state (pos, next_position, K/V bits) must equal the oracle's
bit-exactly; decode outputs must be within 2e-3 of the float64 masked
full-history attention on the same inputs.
"""

import numpy as np
import pytest
import torch

import workloads
from workloads import gen
from tests.gpu_util import (TOL, assert_close, check_ring_rows, f64, host_bits, oracle_out,
                            require_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_tiny_window4_twelve_steps():
    """W=4, 12 append+attend steps from empty (fp32, D=16): unfilled, exactly
    full, first overwrite and wrapping phases."""
    import sliding_window_attention_ring_amd as swa
    wl = workloads.TINY
    say("tiny", wl)
    k = gen.tokens(wl, "k", wl.steps)
    v = gen.tokens(wl, "v", wl.steps)
    cache = swa.KVCache("fp32", wl.B, wl.H, wl.D, wl.W)
    kb, vb = host_bits(k), host_bits(v)
    for t in range(wl.steps):
        swa.kv_append(cache, k[:, :, t:t + 1].contiguous().cuda(), v[:, :, t:t + 1].contiguous().cuda())
        q = gen.query(wl, t)
        out = swa.decode_attn(cache, q.cuda())
        got = out.cpu().numpy()
        check_ring_rows(cache, kb, vb, np.array([t + 1]))
        assert swa.validate(cache) == 0
        ref = oracle_out(f64(k[0]), f64(v[0]), f64(q[0]), t + 1, wl.W)
        assert_close(got[0], ref, f"tiny step {t}")
        if t == 0:  # one visible token: the output is its value row, exactly
            np.testing.assert_array_equal(got[0], v[0, :, 0].numpy())


def run_sweep(kind, D, W, T, B=2, H=2, seed=0, layout="ring"):
    import sliding_window_attention_ring_amd as swa
    g = torch.Generator().manual_seed(seed)
    dt = torch.float32 if kind == "fp32" else torch.bfloat16
    N = 4 * W + T
    k = torch.randn((B, H, N, D), generator=g).to(dt)
    v = torch.randn((B, H, N, D), generator=g).to(dt)
    kb, vb = host_bits(k), host_bits(v)
    k64, v64 = f64(k), f64(v)
    cache = swa.KVCache(kind, B, H, D, W, layout=layout)
    n = 0
    while n < 4 * W:
        swa.kv_append(cache, k[:, :, n:n + T].contiguous().cuda(), v[:, :, n:n + T].contiguous().cuda())
        n += T
        q = torch.randn((B, H, D), generator=g).to(dt)
        got = swa.decode_attn(cache, q.cuda()).cpu().numpy()
        check_ring_rows(cache, kb, vb, np.full(B, n))
        assert swa.validate(cache) == 0
        q64 = f64(q)
        for b in range(B):
            assert_close(got[b], oracle_out(k64[b], v64[b], q64[b], n, W), f"{kind} D={D} W={W} T={T} n={n} b={b}")


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 6])
def test_bruteforce_small_windows_fp32(W):
    """Every chunk size T = 1..2W+1 up to 4W tokens (fp32, D=16)."""
    for T in range(1, 2 * W + 2):
        run_sweep("fp32", 16, W, T, seed=W * 100 + T)


@pytest.mark.parametrize("kind,D,W,Ts", [
    ("bf16", 16, 40, [1, 5, 33, 90]),
    ("bf16", 32, 24, [1, 23, 50]),
    ("bf16", 64, 7, [1, 3, 8, 15]),
    ("bf16", 128, 64, [1, 17, 64, 65, 150]),
    ("bf16", 128, 333, [1, 100, 333, 700]),
    ("bf16", 256, 40, [1, 13, 81]),
    ("fp32", 32, 20, [1, 7, 41]),
    ("fp32", 64, 50, [1, 49, 120]),
    ("fp32", 128, 70, [3, 71]),
    ("fp32", 256, 30, [1, 29, 62]),
])
def test_chunked_appends_all_head_dims(kind, D, W, Ts):
    say("sweep", kind, D, W, Ts)
    for T in Ts:
        run_sweep(kind, D, W, T, seed=D + W + T)


def test_ragged_sequences_through_views():
    """Sequences of one batch at different lengths (each prefilled through a
    B=1 view), including an empty one: the empty sequence outputs zeros."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 5, 3, 128, 200
    g = torch.Generator().manual_seed(7)
    lens = [0, 1, 57, 200, 431]
    k = torch.randn((B, H, max(lens), D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, max(lens), D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache("bf16", B, H, D, W)
    for b, n in enumerate(lens):
        if n:
            swa.kv_append(cache.seq_view(b), k[b:b + 1, :, :n].contiguous().cuda(),
                          v[b:b + 1, :, :n].contiguous().cuda())
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    got = swa.decode_attn(cache, q.cuda()).cpu().numpy()
    check_ring_rows(cache, host_bits(k), host_bits(v), np.array(lens))
    assert swa.validate(cache) == 0
    k64, v64, q64 = f64(k), f64(v), f64(q)
    assert not got[0].any()
    for b in range(1, B):
        assert_close(got[b], oracle_out(k64[b], v64[b], q64[b], lens[b], W), f"ragged b={b}")


def test_decode_is_repeatable_and_workspace_reusable():
    """Same inputs twice: identical bits (the workspace carries no state from
    one call to the next)."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 3, 4, 128, 5000
    g = torch.Generator().manual_seed(3)
    k = torch.randn((B, H, W, D), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((B, H, W, D), generator=g).to(torch.bfloat16).cuda()
    cache = swa.KVCache("bf16", B, H, D, W)
    swa.kv_append(cache, k, v)
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16).cuda()
    a = swa.decode_attn(cache, q).clone()
    b = swa.decode_attn(cache, q).clone()
    assert torch.equal(a, b)
    ref = oracle_out(f64(k[1]), f64(v[1]), f64(q[1]), W, W)
    assert_close(a[1].cpu().numpy(), ref, "repeat")


@pytest.mark.parametrize("W", [64, 640])
def test_empty_sequence_single_and_multi_split(W):
    """An empty sequence outputs zeros both when the plan has one split per
    (b, h) (W=64: the decode kernel finishes each (b, h) itself) and when a
    merge kernel runs (W=640)."""
    import sliding_window_attention_ring_amd as swa
    B, H, D = 3, 2, 128
    g = torch.Generator().manual_seed(W)
    lens = [0, 5, W + 3]
    k = torch.randn((B, H, max(lens), D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache("bf16", B, H, D, W)
    for b, n in enumerate(lens):
        if n:
            swa.kv_append(cache.seq_view(b), k[b:b + 1, :, :n].contiguous().cuda(), k[b:b + 1, :, :n].contiguous().cuda())
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    out = swa.decode_attn(cache, q.cuda()).cpu().numpy()
    assert not out[0].any()
    k64, q64 = f64(k), f64(q)
    for b in (1, 2):
        assert_close(out[b], oracle_out(k64[b], k64[b], q64[b], lens[b], W), f"W={W} b={b}")
