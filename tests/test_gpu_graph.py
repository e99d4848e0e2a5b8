"""The decode step under HIP graph capture.

Positions live on the device (next_position), so one captured step --
kv_append(T=1) then decode -- can be replayed for every new token without a
host round trip ([WitCert] "SGLang 生产级落地": the monitor must survive graph
capture and replay).  Each replay is checked bit for bit against the same
step run eagerly on a twin cache, with eager copies and a synchronization
between replays; the steps cross INT8 block commits.
"""

import pytest
import torch

from tests.gpu_util import host_bits, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("kind,W,prefill", [("int8", 256, 250), ("bf16", 200, 390), ("int8_dither", 128, 300)])
def test_captured_step_replays_match_eager(kind, W, prefill):
    import sliding_window_attention_ring_amd as swa
    B, H, D, steps = 3, 4, 128, 20
    g = torch.Generator().manual_seed(21)
    N = prefill + steps
    k = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).cuda()
    qs = torch.randn((steps, B, H, D), generator=g).to(torch.bfloat16).cuda()
    caches = [swa.KVCache(kind, B, H, D, W) for _ in range(2)]
    for c in caches:
        swa.kv_append(c, k[:, :, :prefill].contiguous(), v[:, :, :prefill].contiguous())
    cg, ce = caches
    static_k = torch.empty((B, H, 1, D), dtype=torch.bfloat16, device="cuda")
    static_v = torch.empty_like(static_k)
    static_q = torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")
    out_g = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    cmax_g = torch.empty((B, H), dtype=torch.float32, device="cuda")
    tv_g = torch.empty((B, H), dtype=torch.float32, device="cuda")
    gate_g = torch.empty((B, H), dtype=torch.int32, device="cuda")
    ws_g = cg.workspace()
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        swa.kv_append(cg, static_k, static_v)
        if kind == "int8":
            swa.decode_attn_int8_witness(cg, static_q, out=out_g, cmax=cmax_g, ws=ws_g)
        elif kind == "int8_dither":
            swa.decode_attn_int8_dither(cg, static_q, delta=1e-3, out=out_g, cert=cmax_g, tv=tv_g, gate=gate_g,
                                        ws=ws_g)
        else:
            swa.decode_attn(cg, static_q, out=out_g, ws=ws_g)
    torch.cuda.synchronize()

    for i in range(steps):
        p = prefill + i
        static_k.copy_(k[:, :, p:p + 1])
        static_v.copy_(v[:, :, p:p + 1])
        static_q.copy_(qs[i])
        graph.replay()
        swa.kv_append(ce, k[:, :, p:p + 1].contiguous(), v[:, :, p:p + 1].contiguous())
        if kind == "int8":
            out_e, cmax_e, _ = swa.decode_attn_int8_witness(ce, qs[i])
        elif kind == "int8_dither":
            out_e, cmax_e, tv_e, gate_e = swa.decode_attn_int8_dither(ce, qs[i], delta=1e-3)
        else:
            out_e = swa.decode_attn(ce, qs[i])
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {i}"
        if kind.startswith("int8"):
            assert torch.equal(cmax_g, cmax_e), f"replay {i}"
        if kind == "int8_dither":
            assert torch.equal(tv_g, tv_e) and torch.equal(gate_g, gate_e), f"replay {i}"
            assert torch.equal(cg.k, ce.k) and torch.equal(cg.k_scale, ce.k_scale), f"replay {i}"
        assert torch.equal(cg.next_position, ce.next_position)
        assert (host_bits(cg.pos) == host_bits(ce.pos)).all()
    assert int(cg.next_position[0]) == prefill + steps
    assert swa.validate(cg) == 0
