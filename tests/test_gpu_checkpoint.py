"""Checkpoint and resume.  The cache state is caller-owned tensors (rows,
positions, next_position; INT8 scales, witness or dither keys, staging
rows; the paged block table), so a checkpoint is a copy of them (the
cache record of the page "LLM 機制實驗（五）", section 哪些東西必須一起裁剪:
keys, values, positions and next_position travel together).  A cache
restored from a host copy into fresh device memory must continue exactly
as the original: every later output, bound and state bit for bit.
"""

import pytest
import torch

from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu

STATE = ("k", "v", "pos", "next_position", "k_scale", "v_scale", "witness", "k_stage", "v_stage", "block_table",
         "request_id")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def decode(swa, c, q):
    if c.kind == "bf16":
        return (swa.decode_attn(c, q),)
    if c.kind == "int8":
        return swa.decode_attn_int8_witness(c, q)[:2]
    return swa.decode_attn_int8_dither(c, q, delta=1e-3)


@pytest.mark.parametrize("kind,layout", [("bf16", "ring"), ("int8", "ring"), ("int8", "paged"),
                                         ("int8_dither", "ring"), ("int8_dither", "paged")])
def test_restore_from_host_copy_continues_bit_for_bit(kind, layout):
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 3, 2, 128, 64
    g = torch.Generator().manual_seed(31)
    N = 150
    k = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).cuda()
    qs = torch.randn((20, B, H, D), generator=g).to(torch.bfloat16).cuda()
    rid = torch.tensor([11, 12, 13], dtype=torch.int64) if kind == "int8_dither" else None
    kw = dict(layout=layout, request_id=rid, layer=4) if kind == "int8_dither" else dict(layout=layout)
    a = swa.KVCache(kind, B, H, D, W, **kw)
    swa.kv_append(a, k[:, :, :123].contiguous(), v[:, :, :123].contiguous())
    snapshot = {n: getattr(a, n).cpu().clone() for n in STATE if getattr(a, n, None) is not None}
    b = swa.KVCache(kind, B, H, D, W, **kw)
    for n, t in snapshot.items():
        getattr(b, n).copy_(t)
    b.desc = b._make_desc()  # block_table / request_id contents were replaced in place; pointers unchanged
    for i in range(20):
        p = 123 + i
        for c in (a, b):
            swa.kv_append(c, k[:, :, p:p + 1].contiguous(), v[:, :, p:p + 1].contiguous())
        oa, ob = decode(swa, a, qs[i]), decode(swa, b, qs[i])
        for x, y in zip(oa, ob):
            assert torch.equal(x, y), f"step {i}"
    for n in snapshot:
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    assert swa.validate(b) == 0
