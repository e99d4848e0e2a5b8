"""Positions near the int32 limit.

Positions are int32 and the documented precondition is next_position + T <
2^31.  A cache is filled normally, then every stored position and
next_position is shifted by S, a multiple of W (so every slot and 16-token
block keeps its place and the position invariant still holds), and tokens
are appended until next_position is within W of 2^31 - 1.  After each
append the ring state is compared bit-exactly (positions S + logical
position) and the decode with the oracle on the logical history (attention
depends on relative positions only).  For the dithered INT8 kind the dither
counter carries the absolute position, so the oracle draws the dither at
S + j, and outputs are compared once every visible block was committed
after the shift.
"""

import numpy as np
import pytest
import torch

from oracle import decoder
from tests.gpu_util import (RingView, assert_close, check_dither_decode, check_dither_store, check_int8_decode,
                            check_int8_store, f64, host_bits, oracle_out, request_ids, require_gpu, say)

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 31 - 1
CHUNKS = [1, 7, 16, 33, 40]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


class Unshifted:
    """The cache's tensors with every stored position moved back by S."""

    def __init__(self, cache, S):
        src = RingView(cache) if cache.layout == "paged" else cache
        for name in ("B", "H", "W", "k", "v", "k_scale", "v_scale", "witness", "k_stage", "v_stage"):
            setattr(self, name, getattr(src, name))
        self.layout = "ring"
        pos = cache.pos.clone()
        pos[pos >= 0] -= S
        self.pos, self.next_position = pos, cache.next_position - S


@pytest.mark.parametrize("kind,layout", [("bf16", "ring"), ("bf16", "paged"), ("int8", "ring"),
                                         ("int8_dither", "ring"), ("int8_dither", "paged")])
def test_positions_near_int32_limit(kind, layout):
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 2, 2, 128, 64
    n1 = 3 * W + 5
    total = n1 + sum(CHUNKS)
    S = W * ((LIMIT - total) // W)
    assert S % 16 == 0 and S + total <= LIMIT
    g = torch.Generator().manual_seed(77)
    k = torch.randn((B, H, total, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, total, D), generator=g).to(torch.bfloat16)
    k64, v64 = f64(k), f64(v)
    cache = swa.KVCache(kind, B, H, D, W, layout=layout)
    swa.kv_append(cache, k[:, :, :n1].contiguous().cuda(), v[:, :, :n1].contiguous().cuda())
    live = cache.pos >= 0
    cache.pos[live] += S
    cache.next_position += S
    torch.cuda.synchronize()
    assert swa.validate(cache) == 0
    say(kind, layout, "shifted by", S)
    n = n1
    for T in CHUNKS:
        swa.kv_append(cache, k[:, :, n:n + T].contiguous().cuda(), v[:, :, n:n + T].contiguous().cuda())
        n += T
        assert swa.validate(cache) == 0
        assert host_bits(cache.next_position).tolist() == [S + n] * B
        q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
        q64 = f64(q)
        view = Unshifted(cache, S)
        if kind == "bf16":
            out = swa.decode_attn(cache, q.cuda()).cpu().numpy()
            pos = host_bits(view.pos)
            kk, vv = host_bits(view.k), host_bits(view.v)
            for b in range(B):
                exp = decoder.expected_ring(np.arange(n), W)
                np.testing.assert_array_equal(pos[b], exp)
                lv = np.nonzero(exp >= 0)[0]
                np.testing.assert_array_equal(kk[b][:, lv], host_bits(k[b])[:, exp[lv]])
                np.testing.assert_array_equal(vv[b][:, lv], host_bits(v[b])[:, exp[lv]])
                assert_close(out[b], oracle_out(k64[b], v64[b], q64[b], n, W), f"near-limit bf16 n={n}")
        elif kind == "int8":
            out, cmax, c_all = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
            out, cmax, c_all = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy()
            for b in range(B):
                for h in range(H):
                    check_int8_store(view, b, h, k64[b, h], v64[b, h], n)
                    check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, q64[b, h], k64[b, h], v64[b, h],
                                      n, W, what=f"near-limit n={n}")
        else:
            out, cert, tv, gate = swa.decode_attn_int8_dither(cache, q.cuda(), delta=1e-3)
            out, cert, tv, gate = out.cpu().numpy(), cert.cpu().numpy(), tv.cpu().numpy(), gate.cpu().numpy()
            reqs = request_ids(cache)
            first_post = (n1 // 16)  # the first block committed after the shift
            for b in range(B):
                for h in range(H):
                    check_dither_store(cache, b, h, k64[b, h], v64[b, h], n, position0=S, first_block=first_post)
                    if n - W >= 16 * first_post:
                        check_dither_decode(out[b, h], cert[b, h], b, h, q64[b, h], k64[b, h], v64[b, h], n, W,
                                            reqs[b], cache.layer, 1e-3, tv[b, h], gate[b, h],
                                            what=f"near-limit n={n}", position0=S)
    assert S + n > LIMIT - W
