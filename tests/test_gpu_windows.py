"""Row caches with window sizes that are not multiples of the kernels' tile
sizes (16-row pages, 64-row iteration rounds): W = 37, 1000 and 4097, bf16
and fp32, with ragged histories that leave some sequences unfilled and wrap
others several times, decoded through decode_attn and the fused step, every
(b, h) against the oracle's full-history masked attention ([Lean-SWA] §2.1)."""

import numpy as np
import pytest
import torch

from tests.gpu_util import assert_close, f64, host_bits, oracle_out, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("kind,W,D", [("bf16", 37, 128), ("bf16", 1000, 64), ("bf16", 4097, 128),
                                       ("fp32", 1000, 32), ("fp32", 37, 16), ("bf16", 1000, 16),
                                       ("bf16", 37, 32), ("fp32", 333, 256)])
def test_odd_windows(kind, W, D):
    import sliding_window_attention_ring_amd as swa
    B, H = 3, 2
    dt = torch.float32 if kind == "fp32" else torch.bfloat16
    rng = np.random.default_rng(W + D)
    lens = [int(rng.integers(1, W)), W, int(rng.integers(W + 1, 3 * W))]  # unfilled, exactly full, wrapped
    N = max(lens) + 3
    g = torch.Generator().manual_seed(W)
    k = torch.randn((B, H, N, D), generator=g).to(dt)
    v = torch.randn((B, H, N, D), generator=g).to(dt)
    cache = swa.KVCache(kind, B, H, D, W)
    for b, n in enumerate(lens):
        swa.kv_append(cache.seq_view(b), k[b:b + 1, :, :n].contiguous().cuda(), v[b:b + 1, :, :n].contiguous().cuda())
    ns = list(lens)
    for step in range(4):
        q = torch.randn((B, H, D), generator=g).to(dt)
        if step == 0:
            out = swa.decode_attn(cache, q.cuda())
        else:  # fused steps: every sequence appends its next token
            kn = torch.stack([k[b, :, ns[b]:ns[b] + 1] for b in range(B)]).contiguous()
            vn = torch.stack([v[b, :, ns[b]:ns[b] + 1] for b in range(B)]).contiguous()
            out = swa.decode_step(cache, kn.cuda(), vn.cuda(), q.cuda())
            ns = [n + 1 for n in ns]
        assert swa.validate(cache) == 0
        assert host_bits(cache.next_position).tolist() == ns
        o = out.cpu().numpy()
        for b in range(B):
            ref = oracle_out(f64(k[b]), f64(v[b]), f64(q[b]), ns[b], W)
            assert_close(o[b], ref, f"{kind} W={W} step {step} b={b}")
    say(f"{kind} W={W} D={D} lens {lens} ok")
