"""Numerical extremes the decode must survive (against the oracle):

* sharply peaked softmax: keys scaled x300 so that logits reach ~1e3 (the
  max-subtracted online softmax and the log-sum-exp merge must not overflow
  or lose the winning row), on one split and on several;
* tiny magnitudes: keys and values near 1e-20 (far below N(0, 1), still
  normal in bf16 and float32), where the softmax is uniform and the output is
  the mean of tiny values;
* INT8 blocks with one outlier 100x the rest: the block scale is set by the
  outlier, the other codes collapse towards 0, the quantization error is
  large, and the witness bound must still cover every token's true logit
  error (page "WitCert", section 频带酉性与双层证书).
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import (assert_close, check_dither_decode, check_int8_decode, f64, oracle_out, request_ids,
                            require_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _fill(swa, cache, k, v):
    swa.kv_append(cache, k.cuda().contiguous(), v.cuda().contiguous())


@pytest.mark.parametrize("W", [64, 4096])
def test_peaked_softmax(W):
    import sliding_window_attention_ring_amd as swa
    B, H, D = 2, 4, 128
    n = W + 7
    g = torch.Generator().manual_seed(W)
    k = (torch.randn((B, H, n, D), generator=g) * 300.0).to(torch.bfloat16)
    v = torch.randn((B, H, n, D), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache("bf16", B, H, D, W)
    _fill(swa, cache, k, v)
    out = swa.decode_attn(cache, q.cuda()).cpu().numpy()
    worst = 0.0
    for b in range(B):
        ref = oracle_out(f64(k[b]), f64(v[b]), f64(q[b]), n, W)
        worst = max(worst, assert_close(out[b], ref, f"peaked W={W} b={b}"))
    logits = (f64(k[0, 0, n - W:]) @ f64(q[0, 0])) / np.sqrt(D)
    say(f"peaked W={W}: largest logit gap {np.max(logits) - np.sort(logits)[-2]:.1f}, max abs err {worst:.2e}")


@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_tiny_magnitudes(kind):
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 2, 4, 128, 64
    n = 70
    g = torch.Generator().manual_seed(3)
    k = (torch.randn((B, H, n, D), generator=g) * 1e-20).to(torch.bfloat16)
    v = (torch.randn((B, H, n, D), generator=g) * 1e-20).to(torch.bfloat16)
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache(kind, B, H, D, W)
    _fill(swa, cache, k, v)
    if kind == "bf16":
        out = swa.decode_attn(cache, q.cuda()).cpu().numpy()
        for b in range(B):
            ref = oracle_out(f64(k[b]), f64(v[b]), f64(q[b]), n, W)
            # relative to the values' scale: the output is a mean of values ~1e-20
            assert np.max(np.abs(out[b] - ref)) <= 2e-3 * 1e-20, b
    else:
        out, cmax, c_all = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
        out, cmax, c_all = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy()
        for b in range(B):
            for h in range(H):
                check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, f64(q[b, h]), f64(k[b, h]),
                                  f64(v[b, h]), n, W, "tiny")
    assert swa.validate(cache) == 0


@pytest.mark.parametrize("kind,layout", [("int8", "ring"), ("int8", "paged"), ("int8_dither", "ring")])
def test_int8_outlier_blocks(kind, layout):
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 2, 4, 128, 128
    n = 2 * W + 9
    g = torch.Generator().manual_seed(17)
    k = torch.randn((B, H, n, D), generator=g)
    v = torch.randn((B, H, n, D), generator=g)
    rng = np.random.default_rng(17)
    # one element per 16-token block 100x the rest, in keys and values (larger values would make the fp32
    # accumulation error of the ~300-sized outputs, not the decode, approach the absolute tolerance)
    for b in range(B):
        for h in range(H):
            for blk in range(n // 16):
                r, d = blk * 16 + int(rng.integers(16)), int(rng.integers(D))
                k[b, h, r, d] *= 100.0
                v[b, h, r, (d + 1) % D] *= 100.0
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache(kind, B, H, D, W, layout=layout)
    _fill(swa, cache, k, v)
    if kind == "int8":
        out, cmax, c_all = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
        out, cmax, c_all = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy()
    else:
        out, cmax, tv, gate = (x.cpu().numpy() for x in swa.decode_attn_int8_dither(cache, q.cuda(), delta=1e-3))
    assert swa.validate(cache) == 0
    reqs = request_ids(cache) if kind == "int8_dither" else None
    for b in range(B):
        for h in range(H):
            if kind == "int8":
                check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, f64(q[b, h]), f64(k[b, h]),
                                  f64(v[b, h]), n, W, f"outlier {layout}")
            else:
                check_dither_decode(out[b, h], cmax[b, h], b, h, f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), n, W,
                                    reqs[b], cache.layer, 1e-3, tv[b, h], gate[b, h], what=f"outlier {layout}")
    say(f"outlier blocks ({kind}, {layout}): bound up to {float(np.max(cmax)):.2f}")
