"""Seeded fuzz of mixed operations against per-sequence oracle histories:
appends of random sizes (whole batch or one sequence through a view),
truncations (exact or fallback), fused decode steps and decodes, on bf16,
fp32 and INT8 caches of both layouts, with one or several splits per (b, h).
After every operation the ring state is compared bit-exactly and every
decode output with the oracle."""

import os

import numpy as np
import pytest
import torch

from oracle import reuse
from tests.gpu_util import (assert_close, check_dither_decode, check_dither_store, check_int8_decode,
                            check_int8_store, check_ring_rows, f64, host_bits, oracle_out, request_ids, require_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("kind,layout,W,seed,D", [("bf16", "ring", 48, 1, 128), ("bf16", "paged", 64, 2, 128),
                                                  ("int8", "ring", 64, 3, 128), ("int8", "paged", 48, 4, 128),
                                                  ("int8_dither", "ring", 48, 5, 128),
                                                  ("int8_dither", "paged", 64, 6, 128),
                                                  # several splits per (b, h) in the decode plans
                                                  ("bf16", "paged", 1024, 7, 128), ("int8", "ring", 1024, 8, 128),
                                                  ("int8_dither", "paged", 1024, 9, 128),
                                                  ("bf16", "ring", 2048, 10, 128), ("int8", "paged", 2048, 11, 128),
                                                  ("int8_dither", "ring", 1024, 12, 128),
                                                  # the other head dims of the row kinds (32 rows per wave load
                                                  # over two pages at D = 16; 4 and 32 splits at D = 32 and 256)
                                                  ("bf16", "paged", 96, 13, 16), ("bf16", "ring", 1024, 14, 32),
                                                  ("bf16", "ring", 1024, 15, 256),
                                                  # fp32 rows: one split on an odd ring, several on a paged pool
                                                  ("fp32", "ring", 33, 16, 64), ("fp32", "paged", 1024, 17, 128)])
def test_mixed_operation_fuzz(kind, layout, W, seed, D):
    import sliding_window_attention_ring_amd as swa
    rng = np.random.default_rng(seed)
    g = torch.Generator().manual_seed(seed)
    B, H = 3, 2
    cache = swa.KVCache(kind, B, H, D, W, layout=layout)
    dt = torch.float32 if kind == "fp32" else torch.bfloat16  # the cache's input dtype
    hist_k = [torch.empty((H, 0, D), dtype=dt) for _ in range(B)]
    hist_v = [torch.empty((H, 0, D), dtype=dt) for _ in range(B)]

    def check_outputs(op, q, outs, ns, step):
        """Every (b, h) output (and bound) of a decode or fused step against the oracle."""
        q64 = f64(q)
        what = f"op {op}{' (step)' if step else ''}"
        if kind == "int8_dither":
            out, cert, tv, gate = (x.cpu().numpy() for x in outs)
            reqs = request_ids(cache)
            for b in range(B):
                for h in range(H):
                    if ns[b] == 0:
                        assert not out[b, h].any() and cert[b, h] == 0
                        continue
                    check_dither_decode(out[b, h], cert[b, h], b, h, q64[b, h], f64(hist_k[b][h]),
                                        f64(hist_v[b][h]), ns[b], W, reqs[b], cache.layer, 1e-3, tv[b, h],
                                        gate[b, h], what=what)
        elif kind == "int8":
            out, cmax = outs[0].cpu().numpy(), outs[1].cpu().numpy()
            c_all = None if step else outs[2].cpu().numpy()
            for b in range(B):
                for h in range(H):
                    check_int8_decode(out[b, h], cmax[b, h], None if c_all is None else c_all[b, h], b, h,
                                      q64[b, h], f64(hist_k[b][h]), f64(hist_v[b][h]), ns[b], W, what=what)
        else:
            out = outs[0].cpu().numpy()
            for b in range(B):
                if ns[b] == 0:
                    assert not out[b].any()
                else:
                    assert_close(out[b], oracle_out(f64(hist_k[b]), f64(hist_v[b]), q64[b], ns[b], W), what)

    for op in range(40):
        r = rng.random()
        if r < 0.45:  # whole-batch append
            T = max(1, int(rng.choice([1, 1, 1, 2, 15, 16, 17, W - 1, W + 5, 2 * W + 3])))  # T >= 1 (W = 1)
            k = torch.randn((B, H, T, D), generator=g).to(dt)
            v = torch.randn((B, H, T, D), generator=g).to(dt)
            swa.kv_append(cache, k.cuda(), v.cuda())
            for b in range(B):
                hist_k[b] = torch.cat([hist_k[b], k[b]], dim=1)
                hist_v[b] = torch.cat([hist_v[b], v[b]], dim=1)
        elif r < 0.7:  # one sequence through a view
            b = int(rng.integers(B))
            T = int(rng.integers(1, 2 * W))
            k = torch.randn((1, H, T, D), generator=g).to(dt)
            v = torch.randn((1, H, T, D), generator=g).to(dt)
            swa.kv_append(cache.seq_view(b), k.cuda(), v.cuda())
            hist_k[b] = torch.cat([hist_k[b], k[0]], dim=1)
            hist_v[b] = torch.cat([hist_v[b], v[0]], dim=1)
        elif r < 0.8 and rng.random() < 0.5:  # fused decode step: one token per sequence, then the decode
            k = torch.randn((B, H, 1, D), generator=g).to(dt)
            v = torch.randn((B, H, 1, D), generator=g).to(dt)
            q = torch.randn((B, H, D), generator=g).to(dt)
            if kind in ("bf16", "fp32"):
                outs = (swa.decode_step(cache, k.cuda(), v.cuda(), q.cuda()),)
            elif kind == "int8":
                outs = swa.decode_step_int8(cache, k.cuda(), v.cuda(), q.cuda(), want_tv=True)
            else:
                outs = swa.decode_step_int8(cache, k.cuda(), v.cuda(), q.cuda(), delta=1e-3, want_tv=True)
            for b in range(B):
                hist_k[b] = torch.cat([hist_k[b], k[b]], dim=1)
                hist_v[b] = torch.cat([hist_v[b], v[b]], dim=1)
            check_outputs(op, q, outs, [hk.shape[1] for hk in hist_k], step=True)
        elif r < 0.8:  # truncation
            ns = [h.shape[1] for h in hist_k]
            cuts = [int(rng.integers(0, n + 1)) for n in ns]
            ok = swa.kv_truncate(cache, torch.tensor(cuts, dtype=torch.int32, device="cuda")).cpu().numpy()
            for b in range(B):
                assert bool(ok[b]) == reuse.truncation_exact(ns[b], cuts[b], W, int8=kind.startswith("int8"))
                if ok[b]:
                    hist_k[b] = hist_k[b][:, :cuts[b]]
                    hist_v[b] = hist_v[b][:, :cuts[b]]
        # state check after every operation
        assert swa.validate(cache) == 0, f"op {op}"
        ns = [h.shape[1] for h in hist_k]
        if kind == "int8":
            for b in range(B):
                for h in range(H):
                    check_int8_store(cache, b, h, f64(hist_k[b][h]), f64(hist_v[b][h]), ns[b])
        elif kind == "int8_dither":
            for b in range(B):
                for h in range(H):
                    check_dither_store(cache, b, h, f64(hist_k[b][h]), f64(hist_v[b][h]), ns[b])
        else:
            N = max(max(ns), 1)
            kb = np.zeros((B, H, N, D), dtype=np.float32 if kind == "fp32" else np.uint16)
            vb = np.zeros_like(kb)
            for b in range(B):
                kb[b, :, :ns[b]] = host_bits(hist_k[b])
                vb[b, :, :ns[b]] = host_bits(hist_v[b])
            check_ring_rows(cache, kb, vb, np.array(ns))
        if rng.random() < 0.6:  # decode
            q = torch.randn((B, H, D), generator=g).to(dt)
            if kind == "int8_dither":
                outs = swa.decode_attn_int8_dither(cache, q.cuda(), delta=1e-3)
            elif kind == "int8":
                outs = swa.decode_attn_int8_witness(cache, q.cuda(), want_c_all=True)
            else:
                outs = (swa.decode_attn(cache, q.cuda()),)
            check_outputs(op, q, outs, ns, step=False)


def random_configurations(seed: int, n: int):
    """n random (kind, layout, W, seed, D) for the fuzz above: every kind and
    layout, windows from 1 slot to 2048 (odd ones on bf16 rings), every head
    dim of the row kinds."""
    rng = np.random.default_rng(seed)
    for _ in range(n):
        kind = str(rng.choice(["bf16", "int8", "int8_dither"]))
        layout = str(rng.choice(["ring", "paged"]))
        if kind == "bf16":
            D = int(rng.choice([16, 32, 64, 128, 256]))
            if layout == "ring":
                W = int(rng.choice([1, 2, 3, 5, 17, 33, 48, 100, 513, 1024, 2047]))
            else:
                W = int(rng.choice([16, 32, 48, 64, 96, 160, 512, 1024, 2048]))
        else:
            D = 128
            W = int(rng.choice([16, 32, 48, 64, 96, 160, 512, 1024, 2048]))
        yield kind, layout, W, int(rng.integers(1000, 10 ** 6)), D


def test_random_configuration_fuzz():
    """The mixed-operation fuzz over random configurations: 8 by default;
    SWA_FUZZ_CONFIGS=<n> and SWA_FUZZ_SEED=<seed> run a wider campaign
    (on MI355X: 200 configurations with the default seed, 222 with seed
    777, 330 with seed 4242, 420 with seed 9001 and 420 with seed 31337
    passed)."""
    n = int(os.environ.get("SWA_FUZZ_CONFIGS", "8"))
    seed = int(os.environ.get("SWA_FUZZ_SEED", "20261202"))
    for i, cfg in enumerate(random_configurations(seed, n)):
        print(f"fuzz configuration {i}: kind={cfg[0]} layout={cfg[1]} W={cfg[2]} seed={cfg[3]} D={cfg[4]}",
              flush=True)
        test_mixed_operation_fuzz(*cfg)
