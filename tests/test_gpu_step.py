"""The fused decode steps (decode_step_int8, decode_step): one token
appended per sequence and the decode in one launch, plus the merge launch
when the plan has several splits per (b, h).

Its result must be bit for bit that of kv_append(T=1) followed by the
separate decode (decode_attn_int8_witness_tv, or decode_attn_int8_dither):
every output, bound, TV value and gate, and the whole cache state (codes,
scales, witness, staging rows, slot positions, next_position), after every
step, on twin caches.  Ragged prefills make different sequences complete
their blocks at different steps; the steps wrap the ring.  Shapes with
B*H at or above the split target (one work-group per CU for INT8, four
for the dithered kind) have one split per (b, h); long-window shapes have
several, so the block a token completes is committed by the split that
decodes it and the staging row by split 0.  A few decodes are also checked
against the oracle, and a graph-captured step is replayed.
"""

import numpy as np
import pytest
import torch

from tests.gpu_util import check_int8_decode, check_int8_store, f64, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def state(c):
    names = ["k", "v", "k_scale", "v_scale", "k_stage", "v_stage", "pos", "next_position"]
    if c.kind == "int8":
        names.append("witness")
    return {n: host_bits(getattr(c, n)).copy() for n in names}


def twins(kind, B, H, W, layout, lens, seed):
    import sliding_window_attention_ring_amd as swa
    g = torch.Generator().manual_seed(seed)
    N = max(lens) + 64
    k = torch.randn((B, H, N, 128), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, N, 128), generator=g).to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = swa.KVCache(kind, B, H, 128, W, layout=layout)
        # rows never written would hold different garbage in the twins: start
        # from zeros, so a stray write by either path still shows
        for name in ("k", "v", "k_scale", "v_scale", "witness", "k_stage", "v_stage"):
            if getattr(c, name) is not None:
                getattr(c, name).zero_()
        for b, n in enumerate(lens):
            if n:
                swa.kv_append(c.seq_view(b), k[b:b + 1, :, :n].contiguous().cuda(), v[b:b + 1, :, :n].contiguous().cuda())
        caches.append(c)
    return caches, k, v, g


def separate(swa, c, kn, vn, q, tau, delta):
    swa.kv_append(c, kn, vn)
    if c.kind == "int8":
        out, cmax, tv, gate, _ = swa.decode_attn_int8_witness_tv(c, q, tau=tau)
    else:
        out, cmax, tv, gate = swa.decode_attn_int8_dither(c, q, delta=delta, tau=tau)
    return out, cmax, tv, gate


@pytest.mark.parametrize("kind,B,H,W,layout", [("int8", 4, 64, 64, "ring"), ("int8", 4, 64, 64, "paged"),
                                               ("int8_dither", 32, 64, 64, "ring"),
                                               ("int8_dither", 32, 64, 64, "paged"),
                                               ("int8", 1, 2, 2048, "ring"), ("int8", 1, 2, 2048, "paged"),
                                               ("int8_dither", 1, 2, 2048, "ring"),
                                               ("int8_dither", 2, 3, 1024, "paged")])
def test_fused_step_equals_append_then_decode(kind, B, H, W, layout):
    import sliding_window_attention_ring_amd as swa
    say("fused step", kind, B, H, W, layout)
    rng = np.random.default_rng(B * H + W)
    lens = [int(x) for x in rng.integers(0, 3 * W, size=B)]
    lens[0] = 13  # one sequence completes its first block at step 3
    (cf, cs), k, v, g = twins(kind, B, H, W, layout, lens, seed=B + W)
    tau, delta = 0.2, 1e-3
    for i in range(40):
        pos = [n + i for n in lens]
        kn = torch.stack([k[b, :, p:p + 1] for b, p in enumerate(pos)]).contiguous().cuda()
        vn = torch.stack([v[b, :, p:p + 1] for b, p in enumerate(pos)]).contiguous().cuda()
        q = torch.randn((B, H, 128), generator=g).to(torch.bfloat16).cuda()
        fo = swa.decode_step_int8(cf, kn, vn, q, tau=tau, delta=delta, want_tv=True)
        so = separate(swa, cs, kn, vn, q, tau, delta)
        for a, b_, name in zip(fo, so, ("out", "cmax", "tv", "gate")):
            assert torch.equal(a, b_), f"step {i}: {name} differs"
        sf, ss = state(cf), state(cs)
        for name in sf:
            np.testing.assert_array_equal(sf[name], ss[name], err_msg=f"step {i}: {name} differs")
        assert host_bits(cf.next_position).tolist() == [n + 1 for n in pos]
    assert swa.validate(cf) == 0
    if kind == "int8":  # the fused path's state and output against the oracle too
        n_after = [n + 40 for n in lens]
        for b in range(min(B, 2)):
            hist_k = f64(k[b, :, :n_after[b]])
            hist_v = f64(v[b, :, :n_after[b]])
            q64 = f64(q.cpu())
            check_int8_store(cf, b, 0, hist_k[0], hist_v[0], n_after[b])
            check_int8_decode(fo[0][b, 0].cpu().numpy(), float(fo[1][b, 0]), None, b, 0, q64[b, 0], hist_k[0],
                              hist_v[0], n_after[b], W, what="fused step")


def test_fused_step_headline_shape_and_graph():
    """B=16, H=32, W=32768 INT8 (one split per (b, h)): a captured fused
    step replayed over 20 tokens, crossing a block commit, equals the eager
    two-launch step on a twin cache each time."""
    import sliding_window_attention_ring_amd as swa
    B, H, W, steps, prefill = 16, 32, 32768, 20, 32768 - 7
    g = torch.Generator(device="cuda").manual_seed(5)
    k = torch.randn((B, H, prefill + steps, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, prefill + steps, 128), generator=g, device="cuda").to(torch.bfloat16)
    qs = torch.randn((steps, B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = swa.KVCache("int8", B, H, 128, W)
        c.k_stage.zero_(); c.v_stage.zero_()
        for c0 in range(0, prefill, 8192):
            c1 = min(prefill, c0 + 8192)
            swa.kv_append(c, k[:, :, c0:c1].contiguous(), v[:, :, c0:c1].contiguous())
        caches.append(c)
    cg, ce = caches
    sk = torch.empty((B, H, 1, 128), dtype=torch.bfloat16, device="cuda")
    sv = torch.empty_like(sk)
    sq = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    cmax = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = cg.workspace()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swa.decode_step_int8(cg, sk, sv, sq, out=out, cmax=cmax, ws=ws)
    torch.cuda.synchronize()
    assert int(cg.next_position[0]) == prefill  # capture does not run the step
    for i in range(steps):
        p = prefill + i
        sk.copy_(k[:, :, p:p + 1]); sv.copy_(v[:, :, p:p + 1]); sq.copy_(qs[i])
        graph.replay()
        swa.kv_append(ce, k[:, :, p:p + 1].contiguous(), v[:, :, p:p + 1].contiguous())
        oe, ce_max, _ = swa.decode_attn_int8_witness(ce, qs[i])
        torch.cuda.synchronize()
        assert torch.equal(out, oe) and torch.equal(cmax, ce_max), f"replay {i}"
        assert torch.equal(cg.next_position, ce.next_position)
        if i % 8 == 7 or p % 16 == 15:
            for name in ("k_stage", "v_stage", "pos", "k_scale"):
                assert torch.equal(getattr(cg, name), getattr(ce, name)), (i, name)
    assert int(cg.next_position[0]) == prefill + steps
    assert swa.validate(cg) == 0


@pytest.mark.parametrize("kind,B,H,D,W,layout", [("bf16", 16, 32, 128, 64, "ring"), ("bf16", 16, 32, 128, 64, "paged"),
                                                 ("fp32", 1, 2, 16, 4, "ring"), ("bf16", 1, 2, 64, 4096, "ring"),
                                                 ("bf16", 1, 2, 64, 4096, "paged"), ("fp32", 2, 3, 32, 1024, "ring"),
                                                 ("bf16", 2, 3, 16, 2048, "paged"), ("bf16", 3, 2, 32, 96, "ring"),
                                                 ("fp32", 2, 2, 256, 512, "ring"),
                                                 # 63 heads: the last counter of the step_sync line
                                                 ("bf16", 1, 63, 128, 4096, "paged"),
                                                 # 64 heads: too many for the in-kernel merge's counters,
                                                 # so the several splits go through the merge kernel
                                                 ("bf16", 1, 64, 128, 4096, "ring")])
def test_fused_row_step_equals_append_then_decode(kind, B, H, D, W, layout):
    """decode_step (bf16 / fp32 kinds) against kv_append + decode_attn on twin
    caches, bit for bit in the output and the ring state, over 3W ragged
    steps (at most 40 for long windows).  The shapes with long windows have
    several splits per (b, h), so the row is written by the split whose slots
    hold it, and the splits are merged in the step kernel (up to 63 heads) or
    by the merge launch (64 heads)."""
    import sliding_window_attention_ring_amd as swa
    say("fused row step", kind, B, H, D, W, layout)
    dt = torch.float32 if kind == "fp32" else torch.bfloat16
    rng = np.random.default_rng(B * H + W)
    lens = [int(x) for x in rng.integers(0, 2 * W, size=B)]
    steps = min(3 * W, 40) if W > 64 else 3 * W
    g = torch.Generator().manual_seed(W + D)
    N = max(lens) + steps
    k = torch.randn((B, H, N, D), generator=g).to(dt)
    v = torch.randn((B, H, N, D), generator=g).to(dt)
    caches = []
    for _ in range(2):
        c = swa.KVCache(kind, B, H, D, W, layout=layout)
        c.k.zero_(); c.v.zero_()
        for b, n in enumerate(lens):
            if n:
                swa.kv_append(c.seq_view(b), k[b:b + 1, :, :n].contiguous().cuda(), v[b:b + 1, :, :n].contiguous().cuda())
        caches.append(c)
    cf, cs = caches
    for i in range(steps):
        pos = [n + i for n in lens]
        kn = torch.stack([k[b, :, p:p + 1] for b, p in enumerate(pos)]).contiguous().cuda()
        vn = torch.stack([v[b, :, p:p + 1] for b, p in enumerate(pos)]).contiguous().cuda()
        q = torch.randn((B, H, D), generator=g).to(dt).cuda()
        of = swa.decode_step(cf, kn, vn, q)
        swa.kv_append(cs, kn, vn)
        os_ = swa.decode_attn(cs, q)
        assert torch.equal(of, os_), f"step {i}: out differs"
        for name in ("k", "v", "pos", "next_position"):
            assert torch.equal(getattr(cf, name), getattr(cs, name)), f"step {i}: {name} differs"
    assert swa.validate(cf) == 0


@pytest.mark.parametrize("kind,B,H,W", [("int8", 4, 64, 64), ("int8_dither", 32, 64, 64), ("bf16", 4, 64, 64),
                                         ("int8", 2, 2, 1024), ("int8_dither", 2, 2, 1024), ("bf16", 2, 2, 1024)])
def test_fused_step_mixed_with_other_operations(kind, B, H, W):
    """Fused steps interleaved with truncations, multi-token appends and
    separate decodes on one cache (sharing its workspace); a twin takes the
    same operations with kv_append + the separate decode only.  Every output
    and the whole state must agree bit for bit after every operation.  The
    W=1024 shapes have several splits per (b, h)."""
    import sliding_window_attention_ring_amd as swa
    say("mixed operations", kind, B, H, W)
    rng = np.random.default_rng(99)
    g = torch.Generator().manual_seed(99)
    caches = []
    for _ in range(2):
        c = swa.KVCache(kind, B, H, 128, W)
        for name in ("k", "v", "k_scale", "v_scale", "witness", "k_stage", "v_stage"):
            if getattr(c, name, None) is not None:
                getattr(c, name).zero_()
        caches.append(c)
    cf, cs = caches
    names = ["k", "v", "pos", "next_position"] + (["k_scale", "v_scale", "k_stage", "v_stage"] if kind != "bf16" else []) \
        + (["witness"] if kind == "int8" else [])

    def rows(T):
        k = torch.randn((B, H, T, 128), generator=g).to(torch.bfloat16).cuda()
        v = torch.randn((B, H, T, 128), generator=g).to(torch.bfloat16).cuda()
        return k, v

    def dec(c, q):
        if kind == "bf16":
            return (swa.decode_attn(c, q),)
        if kind == "int8":
            return swa.decode_attn_int8_witness_tv(c, q)[:4]
        return swa.decode_attn_int8_dither(c, q, delta=1e-3)

    for op in range(60):
        r = rng.random()
        q = torch.randn((B, H, 128), generator=g).to(torch.bfloat16).cuda()
        if r < 0.55:  # fused step on one cache, append + decode on the twin
            k, v = rows(1)
            if kind == "bf16":
                of = (swa.decode_step(cf, k, v, q),)
            else:
                of = swa.decode_step_int8(cf, k, v, q, delta=1e-3, want_tv=True)
            swa.kv_append(cs, k, v)
            os_ = dec(cs, q)
            for a, b_ in zip(of, os_):
                assert torch.equal(a, b_), f"op {op}"
        elif r < 0.7:  # multi-token append on both
            k, v = rows(int(rng.integers(2, 40)))
            for c in caches:
                swa.kv_append(c, k, v)
        elif r < 0.8:  # truncation on both
            n = cf.next_position.cpu().numpy()
            cut = torch.tensor([int(rng.integers(0, m + 1)) for m in n], dtype=torch.int32, device="cuda")
            oka, okb = swa.kv_truncate(cf, cut), swa.kv_truncate(cs, cut)
            assert torch.equal(oka, okb)
        else:  # separate decode on both (uses the same workspace as the fused steps)
            for a, b_ in zip(dec(cf, q), dec(cs, q)):
                assert torch.equal(a, b_), f"op {op}"
        for name in names:
            assert torch.equal(getattr(cf, name), getattr(cs, name)), f"op {op}: {name}"
    assert swa.validate(cf) == 0


@pytest.mark.parametrize("kind", ["int8", "int8_dither", "bf16"])
def test_fused_step_several_splits_graph(kind):
    """B=2, H=3, W=1024 (several splits per (b, h)): the fused step and its
    merge launch captured as one graph and replayed over 40 tokens, crossing
    block commits and the ring wrap, equal the eager kv_append + decode on a
    twin cache after every replay (outputs and the whole cache state)."""
    import sliding_window_attention_ring_amd as swa
    B, H, W, steps = 2, 3, 1024, 40
    say("several-split graph", kind)
    lens = [1000, 1030]  # one sequence fills the ring during the replays, the other has wrapped
    N = max(lens) + steps
    g = torch.Generator(device="cuda").manual_seed(11)
    k = torch.randn((B, H, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    qs = torch.randn((steps, B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = swa.KVCache(kind, B, H, 128, W)
        for name in ("k", "v", "k_scale", "v_scale", "witness", "k_stage", "v_stage"):
            if getattr(c, name, None) is not None:
                getattr(c, name).zero_()
        for b, n in enumerate(lens):
            swa.kv_append(c.seq_view(b), k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous())
        caches.append(c)
    cg, ce = caches
    names = ["k", "v", "pos", "next_position"] + (["k_scale", "v_scale", "k_stage", "v_stage"] if kind != "bf16" else []) \
        + (["witness"] if kind == "int8" else [])
    sk = torch.empty((B, H, 1, 128), dtype=torch.bfloat16, device="cuda")
    sv = torch.empty_like(sk)
    sq = torch.empty((B, H, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    cmax = torch.empty((B, H), dtype=torch.float32, device="cuda")
    tv = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gate = torch.empty((B, H), dtype=torch.int32, device="cuda")
    ws = cg.workspace()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        if kind == "bf16":
            swa.decode_step(cg, sk, sv, sq, out=out, ws=ws)
        else:
            swa.decode_step_int8(cg, sk, sv, sq, delta=1e-3, out=out, cmax=cmax, tv=tv, gate=gate, ws=ws)
    torch.cuda.synchronize()
    assert host_bits(cg.next_position).tolist() == lens  # capture does not run the step
    for i in range(steps):
        kn = torch.stack([k[b, :, n + i:n + i + 1] for b, n in enumerate(lens)]).contiguous()
        vn = torch.stack([v[b, :, n + i:n + i + 1] for b, n in enumerate(lens)]).contiguous()
        sk.copy_(kn); sv.copy_(vn); sq.copy_(qs[i])
        graph.replay()
        swa.kv_append(ce, kn, vn)
        if kind == "bf16":
            eo = (swa.decode_attn(ce, qs[i]),)
            go = (out,)
        elif kind == "int8":
            eo = swa.decode_attn_int8_witness_tv(ce, qs[i])[:4]
            go = (out, cmax, tv, gate)
        else:
            eo = swa.decode_attn_int8_dither(ce, qs[i], delta=1e-3)
            go = (out, cmax, tv, gate)
        torch.cuda.synchronize()
        for a, b_ in zip(go, eo):
            assert torch.equal(a, b_), f"replay {i}"
        for name in names:
            assert torch.equal(getattr(cg, name), getattr(ce, name)), f"replay {i}: {name}"
    assert host_bits(cg.next_position).tolist() == [n + steps for n in lens]
    assert swa.validate(cg) == 0


def test_one_workspace_shared_by_caches_of_different_shapes():
    """One caller workspace, filled with 0xFF bytes, serves fused steps on
    three caches whose split plans differ (bf16 B=1 W=1024: 16 splits per
    (b, h); bf16 B=3 W=16384: 43 splits; INT8 B=2 W=2048), interleaved on one
    stream.  The workspace holds only split partials, so each step must equal
    kv_append + the separate decode on a twin that has a workspace of its own
    -- outputs bit for bit, next_position advanced by one every step."""
    import sliding_window_attention_ring_amd as swa
    shapes = [("bf16", 1, 2, 1024, [700]), ("bf16", 3, 2, 16384, [9000, 16384, 20000]),
              ("int8", 2, 2, 2048, [1500, 2047])]
    g = torch.Generator(device="cuda").manual_seed(23)
    pairs = []
    for kind, B, H, W, lens in shapes:
        N = max(lens) + 40
        k = torch.randn((B, H, N, 128), generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn((B, H, N, 128), generator=g, device="cuda").to(torch.bfloat16)
        twin = []
        for _ in range(2):
            c = swa.KVCache(kind, B, H, 128, W)
            for name in ("k", "v", "k_scale", "v_scale", "witness", "k_stage", "v_stage"):
                if getattr(c, name) is not None:  # never-written rows equal in both twins
                    getattr(c, name).zero_()
            for b, n in enumerate(lens):
                swa.kv_append(c.seq_view(b), k[b:b + 1, :, :n].contiguous(), v[b:b + 1, :, :n].contiguous())
            twin.append(c)
        pairs.append((twin, k, v, list(lens)))
    need = max(swa.workspace_bytes(t[0]) for t, _, _, _ in pairs)
    assert len({swa.workspace_bytes(t[0]) for t, _, _, _ in pairs}) == 3
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    say("shared workspace", need)
    for step in range(12):
        for i in (step % 3, (step + 1) % 3, (step + 2) % 3):
            (cf, cs), k, v, lens = pairs[i]
            n = lens
            kn = torch.stack([k[b, :, x:x + 1] for b, x in enumerate(n)]).contiguous()
            vn = torch.stack([v[b, :, x:x + 1] for b, x in enumerate(n)]).contiguous()
            q = torch.randn((cf.B, cf.H, 128), generator=g, device="cuda").to(torch.bfloat16)
            if cf.kind == "bf16":
                got = (swa.decode_step(cf, kn, vn, q, ws=ws),)
                swa.kv_append(cs, kn, vn)
                ref = (swa.decode_attn(cs, q),)
            else:
                got = swa.decode_step_int8(cf, kn, vn, q, want_tv=True, ws=ws)
                ref = separate(swa, cs, kn, vn, q, 0.2, 1e-6)
            for a, b_ in zip(got, ref):
                assert torch.equal(a, b_), f"step {step} cache {i}"
            pairs[i] = ((cf, cs), k, v, [x + 1 for x in n])
            assert host_bits(cf.next_position).tolist() == pairs[i][3], (step, i)
    for (cf, cs), _, _, _ in pairs:
        assert torch.equal(cf.pos, cs.pos) and torch.equal(cf.k, cs.k)
        assert not cf.step_sync.any(), "every fused step leaves its counters zero"
        assert swa.validate(cf) == 0


@pytest.mark.parametrize("kind,B,H,W", [("bf16", 2, 3, 1024), ("bf16", 16, 32, 64), ("int8", 2, 3, 1024),
                                        ("int8_dither", 2, 3, 1024)])
def test_fused_step_with_a_negative_next_position(kind, B, H, W):
    """A violated precondition forced from the host: next_position of sequence
    0 set to -5.  The fused step appends nothing to it, leaves its
    next_position at -5 and writes zeros for its output (bf16 W=1024: splits
    merged in the step kernel; bf16 W=64: one split; INT8: the merge kernel),
    exactly as kv_append + the separate decode do on a twin; sequence 1
    steps normally, and swa_validate reports the bad sequence."""
    import sliding_window_attention_ring_amd as swa
    g = torch.Generator(device="cuda").manual_seed(47)
    n = W - 24
    k = torch.randn((B, H, n + 1, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, n + 1, 128), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = swa.KVCache(kind, B, H, 128, W)
        for name in ("k", "v", "k_scale", "v_scale", "witness", "k_stage", "v_stage"):
            if getattr(c, name, None) is not None:
                getattr(c, name).zero_()
        swa.kv_append(c, k[:, :, :n].contiguous(), v[:, :, :n].contiguous())
        c.next_position[0] = -5
        caches.append(c)
    cf, cs = caches
    kn, vn = k[:, :, n:n + 1].contiguous(), v[:, :, n:n + 1].contiguous()
    if kind == "bf16":
        got = (swa.decode_step(cf, kn, vn, q),)
        swa.kv_append(cs, kn, vn)
        ref = (swa.decode_attn(cs, q),)
    else:
        got = swa.decode_step_int8(cf, kn, vn, q, want_tv=True, delta=1e-3)
        ref = separate(swa, cs, kn, vn, q, 0.2, 1e-3)
    torch.cuda.synchronize()
    for a, b_ in zip(got, ref):
        assert torch.equal(a, b_)
    assert not got[0][0].any(), "the sequence with the violated precondition gets zeros"
    assert got[0][1].abs().sum() > 0
    assert host_bits(cf.next_position).tolist() == [-5, n + 1] + [n + 1] * (B - 2)
    for name in ("k", "v", "pos"):
        assert torch.equal(getattr(cf, name), getattr(cs, name)), name
    assert not cf.step_sync.any(), "every fused step leaves its counters zero"
    assert swa.validate(cf) > 0
