"""GPU parity of prefix reuse (kv_truncate) through the C ABI.

Each sequence of one batch gets a different (n, cut) case; the device
decides exact truncation vs fallback per sequence, which must match the
oracle's rule.  Then new tokens are appended and the ring state and decode
outputs must equal the oracle of the effective history: history[:cut] + new
when truncated, history + new when it had to fall back (sequence unchanged).
"""

import numpy as np
import pytest
import torch

from oracle import reuse
from tests.gpu_util import (assert_close, check_dither_decode, check_dither_store, check_int8_decode,
                            check_int8_store, check_ring_rows, f64, host_bits, request_ids,
                            oracle_out, require_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def build(swa, kind, W, ns, N, seed):
    B, H, D = len(ns), 2, 128
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache(kind, B, H, D, W)
    for b, n in enumerate(ns):
        if n:
            swa.kv_append(cache.seq_view(b), k[b:b + 1, :, :n].contiguous().cuda(),
                          v[b:b + 1, :, :n].contiguous().cuda())
    return cache, k, v, g


def effective(k, v, b, n, cut, ok, new_k, new_v):
    keep = cut if ok else n
    kk = torch.cat([k[b, :, :keep], new_k[b]], dim=1)
    vv = torch.cat([v[b, :, :keep], new_v[b]], dim=1)
    return kk, vv, keep + new_k.shape[2]


def test_truncate_rows():
    import sliding_window_attention_ring_amd as swa
    W = 64
    ns = [30, 64, 100, 50, 100, 10]
    cuts = [10, 0, 99, 50, 0, 11]  # exact, exact (reset), fallback, no-op, exact (reset), fallback (> n)
    cache, k, v, g = build(swa, "bf16", W, ns, 200, seed=1)
    ok = swa.kv_truncate(cache, torch.tensor(cuts, dtype=torch.int32, device="cuda")).cpu().numpy()
    for b, (n, c) in enumerate(zip(ns, cuts)):
        assert bool(ok[b]) == reuse.truncation_exact(n, c, W), (b, n, c)
    assert swa.validate(cache) == 0
    T = 5
    new_k = torch.randn((len(ns), 2, T, 128), generator=g).to(torch.bfloat16)
    new_v = torch.randn((len(ns), 2, T, 128), generator=g).to(torch.bfloat16)
    swa.kv_append(cache, new_k.cuda(), new_v.cuda())
    q = torch.randn((len(ns), 2, 128), generator=g).to(torch.bfloat16)
    out = swa.decode_attn(cache, q.cuda()).cpu().numpy()
    assert swa.validate(cache) == 0
    for b, (n, c) in enumerate(zip(ns, cuts)):
        kk, vv, n_eff = effective(k, v, b, n, c, ok[b], new_k, new_v)
        kb = np.zeros((len(ns),) + tuple(kk.shape), dtype=np.uint16)
        vb = np.zeros_like(kb)
        kb[b], vb[b] = host_bits(kk), host_bits(vv)
        sub = type("V", (), {})()
        sub.B, sub.W = 1, W
        sub.pos, sub.next_position = cache.pos[b:b + 1], cache.next_position[b:b + 1]
        sub.k, sub.v = cache.k[b:b + 1], cache.v[b:b + 1]
        check_ring_rows(sub, kb[b:b + 1], vb[b:b + 1], np.array([n_eff]))
        assert_close(out[b], oracle_out(f64(kk), f64(vv), f64(q[b]), n_eff, W), f"truncate rows b={b}")


def test_truncate_int8():
    import sliding_window_attention_ring_amd as swa
    W = 64
    ns = [40, 40, 40, 100, 48, 40]
    cuts = [32, 35, 20, 100, 0, 16]  # block boundary, staging tail, inside committed block, no-op, reset, boundary
    cache, k, v, g = build(swa, "int8", W, ns, 200, seed=2)
    ok = swa.kv_truncate(cache, torch.tensor(cuts, dtype=torch.int32, device="cuda")).cpu().numpy()
    for b, (n, c) in enumerate(zip(ns, cuts)):
        assert bool(ok[b]) == reuse.truncation_exact(n, c, W, int8=True), (b, n, c)
    assert list(ok) == [1, 1, 0, 1, 1, 1]
    assert swa.validate(cache) == 0
    T = 20
    new_k = torch.randn((len(ns), 2, T, 128), generator=g).to(torch.bfloat16)
    new_v = torch.randn((len(ns), 2, T, 128), generator=g).to(torch.bfloat16)
    swa.kv_append(cache, new_k.cuda(), new_v.cuda())
    q = torch.randn((len(ns), 2, 128), generator=g).to(torch.bfloat16)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
    out, cmax, c_all = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy()
    assert swa.validate(cache) == 0
    q64 = f64(q)
    for b, (n, c) in enumerate(zip(ns, cuts)):
        kk, vv, n_eff = effective(k, v, b, n, c, ok[b], new_k, new_v)
        k64, v64 = f64(kk), f64(vv)
        for h in range(2):
            check_int8_store(cache, b, h, k64[h], v64[h], n_eff)
            check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, q64[b, h], k64[h], v64[h], n_eff, W,
                              what=f"truncate int8 b={b}")


def test_truncate_int8_dither():
    """Tier B follows the INT8 rule; tokens appended after a cut reuse the
    positions, hence the dither stream, of the tokens they replace."""
    import sliding_window_attention_ring_amd as swa
    W = 64
    ns = [40, 40, 40, 100, 48, 40]
    cuts = [32, 35, 20, 100, 0, 16]
    cache, k, v, g = build(swa, "int8_dither", W, ns, 200, seed=4)
    ok = swa.kv_truncate(cache, torch.tensor(cuts, dtype=torch.int32, device="cuda")).cpu().numpy()
    assert list(ok) == [1, 1, 0, 1, 1, 1]
    assert swa.validate(cache) == 0
    T = 20
    new_k = torch.randn((len(ns), 2, T, 128), generator=g).to(torch.bfloat16)
    new_v = torch.randn((len(ns), 2, T, 128), generator=g).to(torch.bfloat16)
    swa.kv_append(cache, new_k.cuda(), new_v.cuda())
    q = torch.randn((len(ns), 2, 128), generator=g).to(torch.bfloat16)
    out, cert, tv, gate = swa.decode_attn_int8_dither(cache, q.cuda(), delta=1e-3)
    out, cert, tv, gate = out.cpu().numpy(), cert.cpu().numpy(), tv.cpu().numpy(), gate.cpu().numpy()
    assert swa.validate(cache) == 0
    q64 = f64(q)
    reqs = request_ids(cache)
    for b, (n, c) in enumerate(zip(ns, cuts)):
        kk, vv, n_eff = effective(k, v, b, n, c, ok[b], new_k, new_v)
        k64, v64 = f64(kk), f64(vv)
        for h in range(2):
            check_dither_store(cache, b, h, k64[h], v64[h], n_eff)
            check_dither_decode(out[b, h], cert[b, h], b, h, q64[b, h], k64[h], v64[h], n_eff, W, reqs[b],
                                cache.layer, 1e-3, tv[b, h], gate[b, h], what=f"truncate dither b={b}")
