"""GPU parity of the INT8 cache with subtractive dither (Tier B), through the
C ABI.

The oracle draws the same Philox-4x32-10 dither from its own implementation
and quantizes in float32 as the method fixes it, so codes, scales and slot
positions must match bit for bit.  Outputs must be within 2e-3 of the
float64 oracle on the dequantized cache s*(code - u).  The certificate must
equal the oracle's up to its float32 pad, and must not be below the true
largest logit error: each check is an event of probability >= 1 - delta, and
delta = 1e-3 here.  The tests cover every append phase (staging only, block
commits, wrap-around, chunks longer than the window), both layouts, the
single-split and merge paths, ragged and empty sequences, zero blocks,
large request ids, and the TV gate.
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import (check_dither_decode, check_dither_store, f64, host_bits, request_ids,
                            require_gpu, say)

pytestmark = pytest.mark.gpu

DELTA = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def make_cache(B, H, W, layout="ring", layer=5, seed=0):
    import sliding_window_attention_ring_amd as swa
    g = torch.Generator().manual_seed(1000 + seed)
    # large 64-bit ids (as int64 bits) so both key words matter
    rid = torch.randint(-(1 << 62), 1 << 62, (B,), generator=g, dtype=torch.int64)
    return swa.KVCache("int8_dither", B, H, 128, W, layout=layout, request_id=rid, layer=layer)


def run(W, Ts, B=2, H=2, total=None, seed=0, layout="ring", check_store=True):
    import sliding_window_attention_ring_amd as swa
    D = 128
    g = torch.Generator().manual_seed(seed)
    total = total or 3 * W + 20
    N = total + max(Ts)
    k = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    k64, v64 = f64(k), f64(v)
    cache = make_cache(B, H, W, layout, seed=seed)
    reqs = request_ids(cache)
    n, i = 0, 0
    while n < total:
        T = Ts[i % len(Ts)]
        i += 1
        swa.kv_append(cache, k[:, :, n:n + T].contiguous().cuda(), v[:, :, n:n + T].contiguous().cuda())
        n += T
        q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
        out, cert, tv, gate = swa.decode_attn_int8_dither(cache, q.cuda(), delta=DELTA)
        out, cert, tv, gate = out.cpu().numpy(), cert.cpu().numpy(), tv.cpu().numpy(), gate.cpu().numpy()
        assert swa.validate(cache) == 0
        q64 = f64(q)
        for b in range(B):
            for h in range(H):
                if check_store:
                    check_dither_store(cache, b, h, k64[b, h], v64[b, h], n)
                check_dither_decode(out[b, h], cert[b, h], b, h, q64[b, h], k64[b, h], v64[b, h], n, W,
                                    reqs[b], cache.layer, DELTA, tv[b, h], gate[b, h], what=f"W={W} n={n}")


@pytest.mark.parametrize("W,Ts", [
    (16, [1]), (16, [3, 5, 16, 17]), (32, [1, 15, 16, 40]), (64, [7, 64, 65, 150]), (256, [1, 100, 600]),
])
def test_dither_phases(W, Ts):
    say("dither", W, Ts)
    run(W, Ts, seed=W + sum(Ts))


@pytest.mark.parametrize("W,Ts", [(32, [5, 16, 33]), (128, [1, 70, 300])])
def test_dither_phases_paged(W, Ts):
    say("dither paged", W, Ts)
    run(W, Ts, seed=7 * W + sum(Ts), layout="paged")


@pytest.mark.parametrize("B,H,W,n", [(1, 2, 2048, 3000), (16, 16, 64, 150), (3, 4, 512, 517)])
def test_dither_split_and_merge_paths(B, H, W, n):
    """(1, 2, 2048): many splits per (b, h) and the merge kernel; (16, 16,
    64): one split, finished in the main kernel; (3, 4, 512): a staging
    tail on top of a full window."""
    import sliding_window_attention_ring_amd as swa
    say("dither paths", B, H, W, n)
    g = torch.Generator().manual_seed(B * 100 + W)
    k = torch.randn((B, H, n, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, n, 128), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H, 128), generator=g).to(torch.bfloat16)
    cache = make_cache(B, H, W, seed=B + W)
    swa.kv_append(cache, k.cuda(), v.cuda())
    out, cert, tv, gate = swa.decode_attn_int8_dither(cache, q.cuda(), delta=DELTA)
    out, cert, tv, gate = out.cpu().numpy(), cert.cpu().numpy(), tv.cpu().numpy(), gate.cpu().numpy()
    k64, v64, q64 = f64(k), f64(v), f64(q)
    reqs = request_ids(cache)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    if len(pairs) > 12:
        pairs = [pairs[i] for i in np.random.default_rng(0).choice(len(pairs), 12, replace=False)]
    for b, h in pairs:
        check_dither_store(cache, b, h, k64[b, h], v64[b, h], n)
        check_dither_decode(out[b, h], cert[b, h], b, h, q64[b, h], k64[b, h], v64[b, h], n, W, reqs[b],
                            cache.layer, DELTA, tv[b, h], gate[b, h], what="paths")


def test_dither_ragged_and_empty():
    """Sequences of different lengths through single-sequence views, one of
    them empty and one inside its first block (staging only)."""
    import sliding_window_attention_ring_amd as swa
    B, H, W, D = 4, 2, 256, 128
    lens = [0, 9, 300, 777]
    g = torch.Generator().manual_seed(3)
    cache = make_cache(B, H, W, seed=3)
    ks, vs = [], []
    for b, n in enumerate(lens):
        k = torch.randn((1, H, max(n, 1), D), generator=g).to(torch.bfloat16)
        v = torch.randn((1, H, max(n, 1), D), generator=g).to(torch.bfloat16)
        if n:
            swa.kv_append(cache.seq_view(b), k[:, :, :n].contiguous().cuda(), v[:, :, :n].contiguous().cuda())
        ks.append(f64(k[0]))
        vs.append(f64(v[0]))
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    out, cert, tv, gate = swa.decode_attn_int8_dither(cache, q.cuda(), delta=DELTA)
    out, cert, tv, gate = out.cpu().numpy(), cert.cpu().numpy(), tv.cpu().numpy(), gate.cpu().numpy()
    assert swa.validate(cache) == 0
    reqs = request_ids(cache)
    q64 = f64(q)
    for b, n in enumerate(lens):
        for h in range(H):
            if n == 0:
                assert not out[b, h].any() and cert[b, h] == 0 and tv[b, h] == 0 and gate[b, h] == 0
                continue
            check_dither_store(cache, b, h, ks[b][h], vs[b][h], n)
            check_dither_decode(out[b, h], cert[b, h], b, h, q64[b, h], ks[b][h], vs[b][h], n, W, reqs[b],
                                cache.layer, DELTA, tv[b, h], gate[b, h], what="ragged")


def test_dither_zero_block_and_stream_keys():
    """An all-zero head gets scale 0, codes 0 and a zero certificate.  Another
    request id or layer gives other codes but the same attention within the
    tolerance, and the same id and layer give the same codes bit for bit
    (the stream depends on the five-tuple only)."""
    import sliding_window_attention_ring_amd as swa
    B, H, W, n = 1, 2, 64, 80
    g = torch.Generator().manual_seed(8)
    k = torch.randn((B, H, n, 128), generator=g)
    k[:, 1] = 0
    k = k.to(torch.bfloat16)
    v = torch.randn((B, H, n, 128), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H, 128), generator=g).to(torch.bfloat16)
    outs, codes = [], []
    for rid, layer in [(7, 0), (7, 0), (8, 0), (7, 1)]:
        c = swa.KVCache("int8_dither", B, H, 128, W, request_id=torch.tensor([rid]), layer=layer)
        swa.kv_append(c, k.cuda(), v.cuda())
        out, cert, _, _ = swa.decode_attn_int8_dither(c, q.cuda(), delta=DELTA, want_tv=False)
        assert float(cert[0, 1]) == 0 and not host_bits(c.k[0, 1]).any() and not c.k_scale[0, 1].any()
        outs.append(out.cpu().numpy())
        codes.append(host_bits(c.k[0, 0]).copy())
        k64, v64, q64 = f64(k), f64(v), f64(q)
        for h in range(H):
            check_dither_decode(outs[-1][0, h], float(cert[0, h]), 0, h, q64[0, h], k64[0, h], v64[0, h], n, W,
                                rid, layer, DELTA, what=f"rid={rid} layer={layer}")
    assert np.array_equal(codes[0], codes[1]) and np.array_equal(outs[0], outs[1])
    assert not np.array_equal(codes[0], codes[2]) and not np.array_equal(codes[0], codes[3])
    assert np.max(np.abs(outs[0] - outs[2])) < 0.1


def test_dither_tv_gate():
    """A head whose block holds one huge key gets a coarse scale, so its
    certificate and TV bound are large and the gate fires; ordinary heads
    stay below tau.  tv = NULL gives the same out and cert."""
    import sliding_window_attention_ring_amd as swa
    B, H, W, n = 2, 3, 64, 100
    g = torch.Generator().manual_seed(12)
    k = torch.randn((B, H, n, 128), generator=g)
    k[1, 2, 70, 5] = 400.0
    k = k.to(torch.bfloat16)
    v = torch.randn((B, H, n, 128), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H, 128), generator=g).to(torch.bfloat16)
    cache = make_cache(B, H, W, seed=12)
    swa.kv_append(cache, k.cuda(), v.cuda())
    out, cert, tv, gate = swa.decode_attn_int8_dither(cache, q.cuda(), delta=DELTA, tau=0.2)
    out2, cert2, tv2, gate2 = swa.decode_attn_int8_dither(cache, q.cuda(), delta=DELTA, want_tv=False)
    assert tv2 is None and gate2 is None
    assert torch.equal(out, out2) and torch.equal(cert, cert2)
    gate = gate.cpu().numpy()
    assert gate[1, 2] == 1 and gate.sum() == 1, gate
    k64, v64, q64 = f64(k), f64(v), f64(q)
    reqs = request_ids(cache)
    for b in range(B):
        for h in range(H):
            check_dither_decode(out[b, h].cpu().numpy(), float(cert[b, h]), b, h, q64[b, h], k64[b, h], v64[b, h],
                                n, W, reqs[b], cache.layer, DELTA, float(tv[b, h]), int(gate[b, h]), what="tv")
