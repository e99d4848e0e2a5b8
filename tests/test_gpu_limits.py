"""GPU parity at the largest windows the C ABI accepts.

The decode kernels address one (b, h) region with 32-bit byte offsets, and
the descriptor check rejects a region of 4 GiB or more.  These tests fill one
(b, h) at the largest window below that limit -- bf16 W = 2^24 - 16 (K and V
regions of 4 GiB - 4 KiB) and INT8 W = 33554416 (code regions of 4 GiB -
2 KiB) -- wrap the ring, and take the last step with the fused decode step
(several splits per (b, h), then the merge).

Closed form (softmax definition, [KV-Loop] section 三): every key is zero
except two equal "spike" keys, one in the last slot of the region (the
highest byte offset) and one at the oldest visible position, so every other
visible logit is exactly 0 and the two spikes share the logit L.  The exact
output is then (2 e^L out2 + S) / (2 e^L + N - 2), where out2 is the oracle's
attention over the two spike rows alone and S sums the other N - 2 values,
so |out - out2| <= (N - 2) (max|v| + max|out2|) / (2 e^L), below 1e-10 here
(L = 45.25).  The GPU output is compared with out2 to the usual 2e-3, and the
INT8 bound with the oracle's witness bound of the spike rows.  With dither
(Tier B) the zero rows of the two spike blocks read back as -s u, logits of
order 1e-2 instead of 0, and the spikes' logits differ slightly; out2 then
uses each spike's own logit and the neglected terms stay far below the
tolerance, but the bound is not asserted.
"""

import numpy as np
import pytest
import torch

from oracle import attention, int8 as oint8
from tests.gpu_util import assert_close, f64, fp16_witness_slack, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu

D = 128
SPIKE = 4.0     # spike keys are SPIKE in every dim, the query is 1.0: L = 4 * 128 / sqrt(128)
CHUNK = 1 << 20


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def fill(swa, cache, n, spikes, seed, vdt=torch.bfloat16):
    """Append positions 0..n-1 in chunks: keys zero except SPIKE rows at
    `spikes`, values N(0, 1) bf16.  Returns (max |v|, {position: v row
    (fp64)}, {block index: 16 v rows (fp64)} for the spike blocks)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    vmax, vrows, vblocks = 0.0, {}, {}
    need_blocks = {p // 16 for p in spikes}
    for c0 in range(0, n, CHUNK):
        c1 = min(n, c0 + CHUNK)
        k = torch.zeros((1, 1, c1 - c0, D), dtype=vdt, device="cuda")
        v = torch.randn((1, 1, c1 - c0, D), generator=g, device="cuda").to(vdt)
        for p in spikes:
            if c0 <= p < c1:
                k[0, 0, p - c0] = SPIKE
                vrows[p] = f64(v[0, 0, p - c0])
        for blk in need_blocks:
            if c0 <= blk * 16 and blk * 16 + 16 <= c1:
                vblocks[blk] = f64(v[0, 0, blk * 16 - c0:blk * 16 + 16 - c0])
        vmax = max(vmax, float(v.float().abs().max()))
        swa.kv_append(cache, k, v)
        del k, v
    return vmax, vrows, vblocks


def spike_bound(n_vis, vmax, out2, logit):
    return (n_vis - 2) * (vmax + float(np.max(np.abs(out2)))) / (2.0 * np.exp(logit))


@pytest.mark.parametrize("layout", ["ring", "paged"])
def test_bf16_region_at_4gib(layout):
    import sliding_window_attention_ring_amd as swa
    W = (1 << 24) - 16                      # W * D * 2 bytes = 4 GiB - 4 KiB per (b, h)
    n = W + 5                               # wraps: the window is positions [5, W + 4]
    spikes = [W - 1, 5]                     # slot W - 1 (highest offset) and the oldest visible position
    say("bf16 W", W, "n", n, layout)
    cache = swa.KVCache("bf16", 1, 1, D, W, layout=layout)
    vmax, vrows, _ = fill(swa, cache, n - 1, spikes, seed=41)
    kn = torch.zeros((1, 1, 1, D), dtype=torch.bfloat16, device="cuda")
    vn = torch.randn((1, 1, 1, D), generator=torch.Generator(device="cuda").manual_seed(42),
                     device="cuda").to(torch.bfloat16)
    q = torch.ones((1, 1, D), dtype=torch.bfloat16, device="cuda")
    out = swa.decode_step(cache, kn, vn, q)
    out_sep = swa.decode_attn(cache, q)
    assert torch.equal(out, out_sep)
    assert host_bits(cache.next_position).tolist() == [n]
    assert swa.validate(cache) == 0
    assert int(cache.pos[0, W - 1]) == W - 1 and int(cache.pos[0, 4]) == n - 1
    if layout == "paged":  # the spike rows sit in shuffled pages anywhere in the 4 GiB pools
        say("pages of the spike slots", [int(cache.block_table[0, p % W // 16]) for p in spikes])
    kk = np.full((2, D), SPIKE)
    out2 = attention.plain_attention(np.ones(D), kk, np.stack([vrows[p] for p in spikes]))
    logit = SPIKE * D / np.sqrt(D)
    bound = spike_bound(W, max(vmax, float(vn.float().abs().max())), out2, logit)
    assert bound < 1e-10
    err = assert_close(out.cpu().numpy()[0, 0], out2, "bf16 region at 4 GiB")
    say(f"bf16 W={W}: max abs err {err:.2e} (neglected terms <= {bound:.1e})")
    del cache


@pytest.mark.parametrize("kind,layout", [("int8", "ring"), ("int8_dither", "ring"), ("int8", "paged")])
def test_int8_region_at_4gib(kind, layout):
    import sliding_window_attention_ring_amd as swa
    W = 33554416                            # W * D code bytes = 4 GiB - 2 KiB per (b, h)
    n = W + 21                              # wraps; window [21, W + 20]; 5 staged tokens after the step
    spikes = [W - 1, 40]                    # the last slot of the ring and a block near its start
    say(kind, "W", W, "n", n, layout)
    cache = swa.KVCache(kind, 1, 1, D, W, layout=layout)
    vmax, _, vblocks = fill(swa, cache, n - 1, spikes, seed=43)
    kn = torch.zeros((1, 1, 1, D), dtype=torch.bfloat16, device="cuda")
    vn = torch.zeros((1, 1, 1, D), dtype=torch.bfloat16, device="cuda")
    q = torch.ones((1, 1, D), dtype=torch.bfloat16, device="cuda")
    if kind == "int8":
        out, cmax, _, _ = swa.decode_step_int8(cache, kn, vn, q)
        out_sep, cmax_sep, c_all = swa.decode_attn_int8_witness(cache, q, want_c_all=True)
    else:
        out, cmax, _, _ = swa.decode_step_int8(cache, kn, vn, q, delta=1e-6)
        out_sep, cmax_sep, _, _ = swa.decode_attn_int8_dither(cache, q, delta=1e-6)
    assert torch.equal(out, out_sep) and torch.equal(cmax, cmax_sep)
    assert host_bits(cache.next_position).tolist() == [n]
    assert swa.validate(cache) == 0
    # the oracle's dequantized spike rows (their own 16-row blocks; zero rows elsewhere)
    kblock = np.zeros((16, D))
    ks, khat, vhat = [], [], []
    for p in spikes:
        kb = kblock.copy()
        kb[p % 16] = SPIKE
        vb = vblocks[p // 16]
        if kind == "int8":
            s, codes = oint8.quantize_block(kb)
            khat.append(oint8.dequantize(codes, s)[p % 16])
            sv, vcodes = oint8.quantize_block(vb)
            vhat.append(oint8.dequantize(vcodes, sv)[p % 16])
            ks.append(kb[p % 16])
        else:
            from oracle import dither as odither
            req = int(cache.request_id[0])
            u = odither.dither(req, cache.layer, 0, (p // 16) * 16 + np.arange(16), D)
            s, codes = odither.quantize_block(kb, u)
            khat.append(odither.dequantize(codes, s, u)[p % 16])
            sv, vcodes = odither.quantize_block(vb, u)
            vhat.append(odither.dequantize(vcodes, sv, u)[p % 16])
            ks.append(kb[p % 16])
    khat, vhat, ks = np.stack(khat), np.stack(vhat), np.stack(ks)
    logits = khat @ np.ones(D) / np.sqrt(D)
    out2 = attention.plain_attention(np.ones(D), khat, vhat)
    n_vis = W
    if kind == "int8":
        # equal spike logits; the other logits are exactly 0 (zero blocks have s = 0)
        assert logits[0] == logits[1]
        bound = spike_bound(n_vis, vmax, out2, logits[0])
        assert bound < 1e-10
    err = assert_close(out.cpu().numpy()[0, 0], out2, f"{kind} region at 4 GiB")
    e_true = np.abs((ks - khat) @ np.ones(D)) / np.sqrt(D)
    cm = float(cmax[0, 0])
    assert cm >= float(np.max(e_true)), (cm, e_true)
    if kind == "int8":
        c_or = [oint8.witness_bound(np.ones(D), oint8.band_norms(ks[i] - khat[i])) for i in range(2)]
        # The spike residuals are ~1e-7, in fp16's subnormal range (see fp16_witness_slack).
        assert cm <= (max(c_or) + fp16_witness_slack(np.ones(D))) * (1 + 2.0 ** -9), (cm, c_or)
        ca = c_all.cpu().numpy()[0, 0]  # slot-indexed in both layouts
        for i, p in enumerate(spikes):
            assert ca[p % W] >= e_true[i]
        zero = np.ones(W, dtype=bool)
        zero[[p % W for p in spikes]] = False
        assert not np.any(ca[zero]), "zero-key tokens have c_t = 0"
    say(f"{kind} W={W}: max abs err {err:.2e}, bound {cm:.3e} >= true {np.max(e_true):.3e}")
    del cache


@pytest.mark.parametrize("B,H", [(65535, 1), (1, 65535)])
def test_row_cache_at_the_grid_limits(B, H):
    """B or H at 65535, the largest the descriptor accepts (grid dimension
    limits): fp32, D=16, W=4, six fused steps from an empty cache (unfilled,
    full, overwritten); 64 sampled (b, h) pairs per step against the oracle's
    full-history masked attention, the ring state everywhere through
    swa_validate."""
    import sliding_window_attention_ring_amd as swa
    W, steps, Dd = 4, 6, 16
    say("row cache grid limits", B, H)
    g = torch.Generator(device="cuda").manual_seed(B + 7 * H)
    k = torch.randn((B, H, steps, Dd), generator=g, device="cuda")
    v = torch.randn((B, H, steps, Dd), generator=g, device="cuda")
    qs = torch.randn((steps, B, H, Dd), generator=g, device="cuda")
    cache = swa.KVCache("fp32", B, H, Dd, W)
    rng = np.random.default_rng(B + H)
    for t in range(steps):
        out = swa.decode_step(cache, k[:, :, t:t + 1].contiguous(), v[:, :, t:t + 1].contiguous(), qs[t])
        assert swa.validate(cache) == 0
        idx = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(64)]
        o = out.cpu().numpy()
        for b, h in idx:
            ref = attention.masked_attention(f64(qs[t, b, h]), np.arange(t + 1), f64(k[b, h, :t + 1]),
                                             f64(v[b, h, :t + 1]), t, W)
            assert_close(o[b, h], ref, f"grid limits B={B} H={H} t={t} b={b} h={h}")
    assert host_bits(cache.next_position).tolist() == [steps] * B


def test_int8_cache_at_the_head_limit():
    """H = 65535 INT8 heads (one sequence, W = 16, D = 128): 18 fused steps
    from an empty cache commit one block for every head at step 16 (131070
    quantize tasks in the step kernels); sampled heads against the oracle's
    INT8 decode with their bound checked, stores checked bit-exactly."""
    import sliding_window_attention_ring_amd as swa
    from tests.gpu_util import check_int8_decode, check_int8_store
    B, H, W, steps = 1, 65535, 16, 18
    g = torch.Generator(device="cuda").manual_seed(99)
    k = torch.randn((B, H, steps, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, steps, D), generator=g, device="cuda").to(torch.bfloat16)
    qs = torch.randn((steps, B, H, D), generator=g, device="cuda").to(torch.bfloat16)
    cache = swa.KVCache("int8", B, H, D, W)
    rng = np.random.default_rng(5)
    for t in range(steps):
        out, cmax, _, _ = swa.decode_step_int8(cache, k[:, :, t:t + 1].contiguous(), v[:, :, t:t + 1].contiguous(),
                                               qs[t])
        assert swa.validate(cache) == 0
        if t in (0, 14, 15, 16, 17):
            o, cm = out.cpu().numpy(), cmax.cpu().numpy()
            for h in [0, H - 1] + [int(x) for x in rng.integers(H, size=6)]:
                k64, v64 = f64(k[0, h, :t + 1]), f64(v[0, h, :t + 1])
                check_int8_decode(o[0, h], cm[0, h], None, 0, h, f64(qs[t, 0, h]), k64, v64, t + 1, W,
                                  f"head limit t={t}")
                if t == steps - 1:
                    check_int8_store(cache, 0, h, k64, v64, t + 1)
    assert host_bits(cache.next_position).tolist() == [steps]
