"""GPU parity of the INT8 cache with the fused witness bound, through the C ABI.

Codes, scales and slot positions bit-exact vs the oracle; stored witnesses
never below the exact band norm; outputs within 2e-3 of the float64 oracle
on the dequantized cache; c_t never below the true logit error for every
visible token (checked per token, never on aggregates), including queries
aligned band by band with a token's residual, where the bound is tight.
"""

import numpy as np
import pytest
import torch

from oracle import int8 as oint8
from tests.gpu_util import check_int8_decode, check_int8_store, f64, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run(W, Ts, B=2, H=2, steps_total=None, seed=0, check_store_every=1, layout="ring"):
    import sliding_window_attention_ring_amd as swa
    D = 128
    g = torch.Generator().manual_seed(seed)
    total = steps_total or 3 * W + 20
    N = total + max(Ts)
    k = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    k64, v64 = f64(k), f64(v)
    cache = swa.KVCache("int8", B, H, D, W, layout=layout)
    n, i = 0, 0
    while n < total:
        T = Ts[i % len(Ts)]
        i += 1
        swa.kv_append(cache, k[:, :, n:n + T].contiguous().cuda(), v[:, :, n:n + T].contiguous().cuda())
        n += T
        q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
        out, cmax, c_all = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
        out, cmax, c_all = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy()
        assert swa.validate(cache) == 0
        q64 = f64(q)
        for b in range(B):
            for h in range(H):
                if i % check_store_every == 0:
                    check_int8_store(cache, b, h, k64[b, h], v64[b, h], n)
                check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, q64[b, h], k64[b, h],
                                  v64[b, h], n, W, what=f"W={W} n={n}")


@pytest.mark.parametrize("W,Ts", [
    (16, [1]), (16, [3, 5, 16, 17]), (32, [1, 15, 16, 40]), (64, [7, 64, 65, 150]),
    (256, [1, 100, 600]),
])
def test_int8_phases(W, Ts):
    say("int8", W, Ts)
    run(W, Ts, seed=W + sum(Ts))


def test_int8_adversarial_aligned_queries():
    """q_b = lambda_b * r_b for one token's residual r (rounded to bf16): the
    GPU bound for that token stays above its true error and is nearly tight."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 1, 2, 128, 64
    g = torch.Generator().manual_seed(42)
    n = 100
    k = torch.randn((B, H, n, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, n, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache("int8", B, H, D, W)
    swa.kv_append(cache, k.cuda(), v.cuda())
    k64, v64 = f64(k), f64(v)
    for tok in [40, 63, 70, 95]:  # quantized tokens in the window [36, 99]
        q = torch.empty((B, H, D))
        for h in range(H):
            blk = tok // 16
            s, codes = oint8.quantize_block(k64[0, h, blk * 16:(blk + 1) * 16])
            r = k64[0, h, tok] - oint8.dequantize(codes[tok % 16], s)
            lam = np.repeat(np.linspace(0.5, 2.0, D // 8), 8)
            q[0, h] = torch.from_numpy(lam * r / np.max(np.abs(r)))
        q = q.to(torch.bfloat16)
        out, cmax, c_all = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
        q64 = f64(q)
        for h in range(H):
            check_int8_decode(out[0, h].cpu().numpy(), float(cmax[0, h]), c_all[0, h].cpu().numpy(), 0, h,
                              q64[0, h], k64[0, h], v64[0, h], n, W, what=f"aligned tok={tok}")
            res = oint8.int8_decode(q64[0, h], k64[0, h], v64[0, h], n, W)
            j = int(np.nonzero(res["positions"] == tok)[0][0])
            ct = float(c_all[0, h, tok % W])
            assert ct >= res["e"][j] and ct <= res["e"][j] * 1.02, (ct, res["e"][j])


def test_int8_zero_blocks_and_exact_multiples():
    """All-zero keys give scale 0, codes 0 and zero witness; keys that are exact
    multiples of a power-of-two scale with absmax 127 quantize without
    residual, so every c_t is 0 and the output equals plain attention."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 1, 2, 128, 32
    n = 48
    g = torch.Generator().manual_seed(5)
    kint = torch.randint(-127, 128, (B, H, n, D), generator=g).float()
    kint[..., ::16, 0] = 127
    k = (kint * 2.0 ** -4).to(torch.bfloat16)
    k[:, 1] = 0
    v = torch.randn((B, H, n, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache("int8", B, H, D, W)
    swa.kv_append(cache, k.cuda(), v.cuda())
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
    assert not c_all.any() and not cmax.any()
    assert not host_bits(cache.k[0, 1]).any() and not cache.k_scale[0, 1].any()
    k64, v64, q64 = f64(k), f64(v), f64(q)
    for h in range(H):
        check_int8_store(cache, 0, h, k64[0, h], v64[0, h], n)
        check_int8_decode(out[0, h].cpu().numpy(), float(cmax[0, h]), c_all[0, h].cpu().numpy(), 0, h,
                          q64[0, h], k64[0, h], v64[0, h], n, W, what="exact")


def test_int8_tv_bound_and_gate():
    """TV epilogue: tv >= the true total variation between exact-key and
    quantized-key attention weights, tv = tanh(cmax/2) (padded), gate = tv >
    tau; a head whose block holds one huge key (coarse scale, forced from the
    host) must raise the gate while ordinary heads stay below tau.  Outputs
    and cmax equal those of decode_attn_int8_witness bit for bit."""
    import sliding_window_attention_ring_amd as swa
    from oracle import tv as otv
    B, H, D, W, n = 2, 3, 128, 64, 100
    g = torch.Generator().manual_seed(11)
    k = torch.randn((B, H, n, D), generator=g)
    k[1, 2, 70, 5] = 400.0  # outlier: block 4 of (b=1, h=2) gets a coarse scale
    k = k.to(torch.bfloat16)
    v = torch.randn((B, H, n, D), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache("int8", B, H, D, W)
    swa.kv_append(cache, k.cuda(), v.cuda())
    out, cmax, tvb, gate, _ = swa.decode_attn_int8_witness_tv(cache, q.cuda(), tau=0.2)
    out2, cmax2, _ = swa.decode_attn_int8_witness(cache, q.cuda())
    assert torch.equal(out, out2) and torch.equal(cmax, cmax2)
    tvb, gate, cmax = tvb.cpu().numpy(), gate.cpu().numpy(), cmax.cpu().numpy()
    k64, v64, q64 = f64(k), f64(v), f64(q)
    for b in range(B):
        for h in range(H):
            r = otv.int8_attention_tv(q64[b, h], k64[b, h], v64[b, h], n, W)
            t = float(tvb[b, h])
            assert t >= r["tv"], (b, h, t, r["tv"])
            assert t >= np.tanh(0.5 * float(cmax[b, h])) * (1 - 2.0 ** -22)
            assert t <= r["bound"] * (1 + 2.0 ** -8) + 1e-7, (t, r["bound"])
            assert gate[b, h] == (1 if t > 0.2 else 0)
            assert gate[b, h] == (1 if (b, h) == (1, 2) else 0)


@pytest.mark.parametrize("W", [16, 512])
def test_int8_empty_and_short_sequences(W):
    """n = 0 gives zero output and cmax 0; n < 16 (staging only) gives exact
    attention over the staged rows with cmax 0 -- on the single-split path
    (W=16) and with a merge kernel (W=512)."""
    import sliding_window_attention_ring_amd as swa
    B, H, D = 3, 2, 128
    g = torch.Generator().manual_seed(W + 1)
    lens = [0, 7, 40]
    k = torch.randn((B, H, max(lens), D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, max(lens), D), generator=g).to(torch.bfloat16)
    cache = swa.KVCache("int8", B, H, D, W)
    for b, n in enumerate(lens):
        if n:
            swa.kv_append(cache.seq_view(b), k[b:b + 1, :, :n].contiguous().cuda(), v[b:b + 1, :, :n].contiguous().cuda())
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    out, cmax, c_all = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
    out, cmax, c_all = out.cpu().numpy(), cmax.cpu().numpy(), c_all.cpu().numpy()
    assert not out[0].any() and not cmax[0].any() and not c_all[0].any()
    assert not cmax[1].any()
    k64, v64, q64 = f64(k), f64(v), f64(q)
    for b in (1, 2):
        for h in range(H):
            check_int8_decode(out[b, h], cmax[b, h], c_all[b, h], b, h, q64[b, h], k64[b, h], v64[b, h], lens[b], W,
                              what=f"W={W}")


def test_int8_forced_corruption_is_detected():
    """Failure detection forced from the host: zeroed witnesses make the
    kernel report cmax = 0, and the per-token soundness check rejects it;
    a block's key scale forced up moves the output away from the oracle and
    the parity check rejects that."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W, n = 1, 2, 128, 64, 90
    g = torch.Generator().manual_seed(23)
    k = torch.randn((B, H, n, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, n, D), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    k64, v64, q64 = f64(k), f64(v), f64(q)
    cache = swa.KVCache("int8", B, H, D, W)
    swa.kv_append(cache, k.cuda(), v.cuda())
    out, cmax, _ = swa.decode_attn_int8_witness(cache, q.cuda())
    check_int8_decode(out[0, 0].cpu().numpy(), float(cmax[0, 0]), None, 0, 0, q64[0, 0], k64[0, 0], v64[0, 0], n, W)
    cache.witness.zero_()
    out, cmax, _ = swa.decode_attn_int8_witness(cache, q.cuda())
    assert float(cmax.abs().max()) == 0.0
    with pytest.raises(AssertionError):
        check_int8_decode(out[0, 0].cpu().numpy(), float(cmax[0, 0]), None, 0, 0, q64[0, 0], k64[0, 0],
                          v64[0, 0], n, W)
    cache.k_scale[0, 0, 2] *= 4  # block of positions 32..47: visible
    out, cmax, _ = swa.decode_attn_int8_witness(cache, q.cuda())
    with pytest.raises(AssertionError):
        check_int8_decode(out[0, 0].cpu().numpy(), 1e30, None, 0, 0, q64[0, 0], k64[0, 0], v64[0, 0], n, W)
