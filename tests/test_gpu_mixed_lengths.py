"""GPU parity of row (bf16/fp32) caches whose sequences have very different
lengths in one batch.

The decode splits each (b, h) into chunks sized for a full cache, so short
and empty sequences leave most of their splits with nothing to read, long
ones spread over many splits merged by the second kernel, and one-split
plans finish each (b, h) in the decode kernel.  These cases cover empty
sequences, one-token and one-block sequences, a ring that has wrapped, one
(b, h) spread over 64 splits, more than 256 sequences, and windows smaller
than a 16-slot block.  Every (b, h) is checked against the oracle's
attention over the last W tokens, and repeated calls must give identical
bits (the merge order is fixed).
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import (assert_close, check_dither_decode, check_int8_decode, check_ring_rows, f64, host_bits,
                            oracle_out, request_ids, require_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _prefill(swa, cache, k, v, lens):
    for b, n in enumerate(lens):
        if n:
            swa.kv_append(cache.seq_view(b), k[b:b + 1, :, :n].contiguous().cuda(),
                          v[b:b + 1, :, :n].contiguous().cuda())


def _check_all(out, k64, v64, q64, lens, W, what):
    for b, n in enumerate(lens):
        if n == 0:
            assert not out[b].any(), f"{what}: empty sequence {b} must output zeros"
            continue
        assert_close(out[b], oracle_out(k64[b], v64[b], q64[b], n, W), f"{what} b={b} len={n}")


@pytest.mark.parametrize("kind,D,layout", [("bf16", 128, "ring"), ("bf16", 128, "paged"), ("fp32", 64, "ring"),
                                           ("bf16", 256, "ring")])
def test_mixed_lengths_decode_and_fused_steps(kind, D, layout):
    """B=9, H=3, W=4096 (ten splits per (b, h)): lengths 0, 1, 15, 16, 17,
    4096, 9000 (wrapped), 300, 2500; decode_attn, then five fused steps
    (every sequence gains a token, the empty one its first)."""
    import sliding_window_attention_ring_amd as swa
    B, H, W, steps = 9, 3, 4096, 5
    lens = [0, 1, 15, 16, 17, 4096, 9000, 300, 2500]
    say("mixed lengths", kind, D, layout)
    g = torch.Generator().manual_seed(D + len(layout))
    N = max(lens) + steps
    dt = torch.bfloat16 if kind == "bf16" else torch.float32
    k = torch.randn((B, H, N, D), generator=g).to(dt)
    v = torch.randn((B, H, N, D), generator=g).to(dt)
    qs = torch.randn((steps + 1, B, H, D), generator=g).to(dt)
    cache = swa.KVCache(kind, B, H, D, W, layout=layout)
    _prefill(swa, cache, k, v, lens)
    k64, v64, q64 = f64(k), f64(v), f64(qs)
    out = swa.decode_attn(cache, qs[0].cuda()).cpu().numpy()
    _check_all(out, k64, v64, q64[0], lens, W, f"decode {kind} {layout}")
    for i in range(steps):
        kn = torch.stack([k[b, :, n + i:n + i + 1] for b, n in enumerate(lens)]).contiguous().cuda()
        vn = torch.stack([v[b, :, n + i:n + i + 1] for b, n in enumerate(lens)]).contiguous().cuda()
        out = swa.decode_step(cache, kn, vn, qs[i + 1].cuda()).cpu().numpy()
        now = [n + i + 1 for n in lens]
        _check_all(out, k64, v64, q64[i + 1], now, W, f"step {i} {kind} {layout}")
        assert host_bits(cache.next_position).tolist() == now
    check_ring_rows(cache, host_bits(k), host_bits(v), np.array([n + steps for n in lens]))
    assert swa.validate(cache) == 0


def test_one_long_sequence_among_short_ones():
    """B=4, H=1, W=131072 with lengths 131072, 1, 0, 17: the long sequence
    is read by 64 splits and merged from all of them, the others by one or
    none; three calls give identical bits."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 4, 1, 128, 131072
    lens = [W, 1, 0, 17]
    g = torch.Generator().manual_seed(41)
    k = torch.randn((B, H, W, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, W, D), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache("bf16", B, H, D, W)
    _prefill(swa, cache, k, v, lens)
    outs = [swa.decode_attn(cache, q.cuda()).clone() for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    _check_all(outs[0].cpu().numpy(), f64(k), f64(v), f64(q), lens, W, "one long pair")


@pytest.mark.parametrize("B,H,W,D", [(300, 2, 64, 16), (2, 1, 4, 16), (257, 1, 512, 32)])
def test_many_sequences_and_tiny_windows(B, H, W, D):
    """More than 256 sequences (one split per (b, h)) and a window of 4 slots,
    less than a 16-slot block.  fp32, random lengths in [0, 3W], every
    (b, h) against the oracle, twice."""
    import sliding_window_attention_ring_amd as swa
    rng = np.random.default_rng(B + W)
    lens = [int(x) for x in rng.integers(0, 3 * W + 1, size=B)]
    lens[0] = 0
    lens[-1] = max(lens[-1], 1)
    say("many sequences / tiny windows", B, H, W, D)
    g = torch.Generator().manual_seed(B * W)
    N = max(lens)
    k = torch.randn((B, H, N, D), generator=g)
    v = torch.randn((B, H, N, D), generator=g)
    q = torch.randn((B, H, D), generator=g)
    cache = swa.KVCache("fp32", B, H, D, W)
    _prefill(swa, cache, k, v, lens)
    a = swa.decode_attn(cache, q.cuda()).clone()
    b_ = swa.decode_attn(cache, q.cuda()).clone()
    assert torch.equal(a, b_)
    _check_all(a.cpu().numpy(), f64(k), f64(v), f64(q), lens, W, f"B={B} W={W}")
    assert swa.validate(cache) == 0


def test_ragged_fused_step_graph():
    """B=6, H=2, W=2048, lengths 0..2100: the fused step (16 splits per
    (b, h), plus the merge launch) captured once and replayed over 24 tokens (the ring of one sequence wraps, the
    empty one fills) equals the eager kv_append + decode_attn on a twin
    cache after every replay, bit for bit, with the whole cache state."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W, steps = 6, 2, 128, 2048, 24
    lens = [0, 3, 700, 2040, 2100, 1500]
    N = max(lens) + steps
    g = torch.Generator(device="cuda").manual_seed(5)
    k = torch.randn((B, H, N, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=g, device="cuda").to(torch.bfloat16)
    qs = torch.randn((steps, B, H, D), generator=g, device="cuda").to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = swa.KVCache("bf16", B, H, D, W)
        c.k.zero_()
        c.v.zero_()
        _prefill(swa, c, k, v, lens)
        caches.append(c)
    cg, ce = caches
    sk = torch.empty((B, H, 1, D), dtype=torch.bfloat16, device="cuda")
    sv = torch.empty_like(sk)
    sq = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    ws = cg.workspace()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swa.decode_step(cg, sk, sv, sq, out=out, ws=ws)
    torch.cuda.synchronize()
    for i in range(steps):
        kn = torch.stack([k[b, :, n + i:n + i + 1] for b, n in enumerate(lens)]).contiguous()
        vn = torch.stack([v[b, :, n + i:n + i + 1] for b, n in enumerate(lens)]).contiguous()
        sk.copy_(kn)
        sv.copy_(vn)
        sq.copy_(qs[i])
        graph.replay()
        swa.kv_append(ce, kn, vn)
        eo = swa.decode_attn(ce, qs[i])
        torch.cuda.synchronize()
        assert torch.equal(out, eo), f"replay {i}"
        for name in ("k", "v", "pos", "next_position"):
            assert torch.equal(getattr(cg, name), getattr(ce, name)), f"replay {i}: {name}"
    assert host_bits(cg.next_position).tolist() == [n + steps for n in lens]
    k64, v64, q64 = f64(k), f64(v), f64(qs[-1])
    _check_all(out.cpu().numpy(), k64, v64, q64, [n + steps for n in lens], W, "graph last replay")
    assert swa.validate(cg) == 0


@pytest.mark.parametrize("kind", ["bf16", "int8", "int8_dither"])
def test_unwritten_partials_are_never_read(kind):
    """A caller's workspace filled with NaN bit patterns (the workspace holds
    only split partials and needs no initialization): with lengths that leave
    most of the planned splits empty, the merge must read only the splits
    that were written this call."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 3, 2, 128, 1024
    lens = [1, 100, W + 37]
    say("NaN workspace", kind)
    g = torch.Generator().manual_seed(19)
    N = max(lens) + 1
    k = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    qs = torch.randn((2, B, H, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache(kind, B, H, D, W)
    _prefill(swa, cache, k, v, lens)
    ws = torch.full((swa.workspace_bytes(cache),), 0xFF, dtype=torch.uint8, device="cuda")
    k64, v64, q64 = f64(k), f64(v), f64(qs)
    if kind == "bf16":
        out = swa.decode_attn(cache, qs[0].cuda(), ws=ws).cpu().numpy()
        _check_all(out, k64, v64, q64[0], lens, W, "NaN workspace decode")
        kn = torch.stack([k[b, :, n:n + 1] for b, n in enumerate(lens)]).contiguous().cuda()
        vn = torch.stack([v[b, :, n:n + 1] for b, n in enumerate(lens)]).contiguous().cuda()
        out = swa.decode_step(cache, kn, vn, qs[1].cuda(), ws=ws).cpu().numpy()
        _check_all(out, k64, v64, q64[1], [n + 1 for n in lens], W, "NaN workspace step")
    elif kind == "int8":
        out, cmax, c_all = swa.decode_attn_int8_witness(cache, qs[0].cuda(), ws=ws, want_c_all=True)
        out, cmax, c_all = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy()
        for b, n in enumerate(lens):
            for h in range(H):
                check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, q64[0, b, h], k64[b, h], v64[b, h], n,
                                  W, "NaN workspace")
    else:
        out, cert, tv, gate = (x.cpu().numpy() for x in swa.decode_attn_int8_dither(cache, qs[0].cuda(),
                                                                                      delta=1e-3, ws=ws))
        reqs = request_ids(cache)
        for b, n in enumerate(lens):
            for h in range(H):
                check_dither_decode(out[b, h], cert[b, h], b, h, q64[0, b, h], k64[b, h], v64[b, h], n, W, reqs[b],
                                    cache.layer, 1e-3, tv[b, h], gate[b, h], what="NaN workspace")
    assert swa.validate(cache) == 0
