"""decode_step_int8_static: the fused INT8 step with its split partials in
the library's static device scratch (for callers that cannot allocate).

Through the C ABI, its results must equal decode_step_int8's bit for bit
(every output, bound, TV value and gate, and the whole cache state) on twin
caches, on two calls in a row, the second with a smaller input, for both
INT8 kinds.  The shapes have several splits per (b, h), so the partials do
go through the scratch.  A shape whose partials exceed the scratch is
rejected on the host with SWA_EWORKSPACE.
"""

import ctypes

import pytest
import torch

from tests.gpu_util import host_bits, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _twins(swa, kind, B, H, W, n, g):
    k = torch.randn((B, H, n + 1, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, n + 1, 128), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = swa.KVCache(kind, B, H, 128, W)
        for name in ("k", "v", "k_scale", "v_scale", "witness", "k_stage", "v_stage"):
            if getattr(c, name) is not None:
                getattr(c, name).zero_()
        swa.kv_append(c, k[:, :, :n].contiguous(), v[:, :, :n].contiguous())
        caches.append(c)
    return caches, k[:, :, n:n + 1].contiguous(), v[:, :, n:n + 1].contiguous(), q


@pytest.mark.parametrize("kind", ["int8", "int8_dither"])
def test_static_scratch_step_equals_workspace_step(kind):
    import sliding_window_attention_ring_amd as swa
    g = torch.Generator(device="cuda").manual_seed(41)
    # (B, H, W, n): the first has 8 splits per (b, h) and commits a block
    # (n = 1007 -> 1008); the second is smaller, with 4 splits.
    for B, H, W, n in [(2, 3, 1024, 1007), (1, 2, 512, 700)]:
        say("static scratch step", kind, B, H, W, n)
        (cs, cw), kn, vn, q = _twins(swa, kind, B, H, W, n, g)
        assert swa.workspace_bytes(cs) > B * H * (128 + 4) * 4  # several splits per (b, h)
        ws = torch.full((swa.workspace_bytes(cw),), 0xFF, dtype=torch.uint8, device="cuda")
        outs = []
        for c, static in ((cs, True), (cw, False)):
            out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
            cmax = torch.empty((B, H), dtype=torch.float32, device="cuda")
            tv = torch.empty((B, H), dtype=torch.float32, device="cuda")
            gate = torch.empty((B, H), dtype=torch.int32, device="cuda")
            if static:
                swa.decode_step_int8_static(c, kn, vn, q, delta=1e-3, out=out, cmax=cmax, tv=tv, gate=gate)
            else:
                swa.decode_step_int8(c, kn, vn, q, delta=1e-3, out=out, cmax=cmax, tv=tv, gate=gate, ws=ws)
            outs.append((out, cmax, tv, gate))
        torch.cuda.synchronize()
        for a, b in zip(*outs):
            assert torch.equal(a, b), (kind, B, H, W, n)
        assert bool(torch.isfinite(outs[0][0]).all())
        names = ["k", "v", "k_scale", "v_scale", "k_stage", "v_stage", "pos", "next_position"]
        if kind == "int8":
            names.append("witness")
        for name in names:
            assert torch.equal(getattr(cs, name), getattr(cw, name)), name
        assert host_bits(cs.next_position).tolist() == [n + 1] * B
        assert not cs.step_sync.any()


def test_oversized_shape_is_rejected_before_any_launch():
    """65535 sequences of 2 heads need 65535*2*528 bytes of partials at one
    split each (69 MB > 16 MiB): SWA_EWORKSPACE, nothing launched."""
    from sliding_window_attention_ring_amd._capi import SwaCacheDesc, lib
    d = SwaCacheDesc(kind=2, B=65535, H=2, D=128, W=16, layout=0, k=0x10000, v=0x20000, pos=0x30000,
                     next_position=0x40000, k_scale=0x50000, v_scale=0x60000, witness=0x70000, k_stage=0x80000,
                     v_stage=0x90000, block_table=None, num_pages=0, request_id=None, layer=0, step_sync=0xE0000)
    assert lib().swa_workspace_bytes(ctypes.byref(d)) > 16 << 20
    a = ctypes.c_void_p(0xA0000)
    assert lib().decode_step_int8_static(ctypes.byref(d), a, a, a, a, a, None, None, 0.2, 0.1, None) == -5


@pytest.mark.parametrize("kind", ["int8", "int8_dither"])
def test_static_scratch_step_under_graph_capture(kind):
    """The callers it is for: one decode_step_int8_static call captured in a
    graph (after a first eager call on the device, which looks the scratch
    address up) and replayed for 20 tokens, across block commits, equals the
    eager decode_step_int8 on a twin after every replay, with eager work and
    a synchronization between the replays."""
    import sliding_window_attention_ring_amd as swa
    B, H, W, n, steps = 2, 3, 1024, 1000, 20
    g = torch.Generator(device="cuda").manual_seed(43)
    k = torch.randn((B, H, n + steps + 1, 128), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, n + steps + 1, 128), generator=g, device="cuda").to(torch.bfloat16)
    qs = torch.randn((steps + 1, B, H, 128), generator=g, device="cuda").to(torch.bfloat16)
    caches = []
    for _ in range(2):
        c = swa.KVCache(kind, B, H, 128, W)
        for name in ("k", "v", "k_scale", "v_scale", "witness", "k_stage", "v_stage"):
            if getattr(c, name) is not None:
                getattr(c, name).zero_()
        swa.kv_append(c, k[:, :, :n].contiguous(), v[:, :, :n].contiguous())
        caches.append(c)
    cg, ce = caches
    sk = k[:, :, n:n + 1].contiguous()
    sv = v[:, :, n:n + 1].contiguous()
    sq = qs[0].clone()
    out = torch.empty((B, H, 128), dtype=torch.float32, device="cuda")
    cmax = torch.empty((B, H), dtype=torch.float32, device="cuda")
    tv = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gate = torch.empty((B, H), dtype=torch.int32, device="cuda")
    args = dict(delta=1e-3, out=out, cmax=cmax, tv=tv, gate=gate)
    swa.decode_step_int8_static(cg, sk, sv, sq, **args)   # first call on the device: eager
    eo = swa.decode_step_int8(ce, sk, sv, sq, delta=1e-3, want_tv=True)
    torch.cuda.synchronize()
    for a, b in zip((out, cmax, tv, gate), eo):
        assert torch.equal(a, b)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swa.decode_step_int8_static(cg, sk, sv, sq, **args)
    torch.cuda.synchronize()
    assert host_bits(cg.next_position).tolist() == [n + 1] * B  # capture does not run the step
    names = ["k", "v", "k_scale", "v_scale", "k_stage", "v_stage", "pos", "next_position"] + \
        (["witness"] if kind == "int8" else [])
    for i in range(1, steps + 1):
        sk.copy_(k[:, :, n + i:n + i + 1])
        sv.copy_(v[:, :, n + i:n + i + 1])
        sq.copy_(qs[i])
        graph.replay()
        eo = swa.decode_step_int8(ce, sk, sv, sq, delta=1e-3, want_tv=True)
        torch.cuda.synchronize()
        for a, b in zip((out, cmax, tv, gate), eo):
            assert torch.equal(a, b), f"replay {i}"
        for name in names:
            assert torch.equal(getattr(cg, name), getattr(ce, name)), f"replay {i}: {name}"
    assert host_bits(cg.next_position).tolist() == [n + steps + 1] * B
