"""GPU parity of the paged layout: pools of 16-token pages addressed through
a per-sequence block table (shuffled page order).  The logical cache -- the
ring read back through the table -- must equal the oracle's window exactly,
and outputs must match the oracle as for the contiguous ring.
"""

import numpy as np
import pytest
import torch

from tests import test_gpu_int8, test_gpu_ring
from tests.gpu_util import assert_close, check_ring_rows, f64, host_bits, oracle_out, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("kind,D,W,Ts", [
    ("fp32", 16, 16, [1, 5, 16, 33]),
    ("bf16", 128, 64, [1, 17, 64, 65, 150]),
    ("bf16", 128, 336, [1, 100, 700]),
    ("bf16", 64, 48, [3, 40]),
    ("bf16", 256, 32, [1, 70]),
    ("bf16", 16, 80, [1, 33, 170]),
    ("bf16", 32, 48, [5, 60]),
    ("fp32", 256, 32, [1, 50]),
])
def test_paged_rows(kind, D, W, Ts):
    for T in Ts:
        test_gpu_ring.run_sweep(kind, D, W, T, seed=D + W + T, layout="paged")


@pytest.mark.parametrize("W,Ts", [(16, [1, 3, 17]), (64, [7, 64, 65, 150]), (256, [1, 100, 600])])
def test_paged_int8(W, Ts):
    test_gpu_int8.run(W, Ts, seed=W + sum(Ts) + 1, layout="paged")


def test_paged_large_pool_custom_table():
    """A pool three times larger than needed, pages picked at random by the
    caller; appends of several sizes then a decode."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 3, 4, 128, 128
    g = torch.Generator().manual_seed(9)
    P = 3 * B * (W // 16)
    table = torch.randperm(P, generator=g)[: B * (W // 16)].reshape(B, W // 16).to(torch.int32)
    cache = swa.KVCache("bf16", B, H, D, W, layout="paged", num_pages=P, block_table=table)
    N = 300
    k = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    n = 0
    for T in [1, 30, 2, 100, 16, 151]:
        swa.kv_append(cache, k[:, :, n:n + T].contiguous().cuda(), v[:, :, n:n + T].contiguous().cuda())
        n += T
    q = torch.randn((B, H, D), generator=g).to(torch.bfloat16)
    out = swa.decode_attn(cache, q.cuda()).cpu().numpy()
    check_ring_rows(cache, host_bits(k), host_bits(v), np.full(B, n))
    assert swa.validate(cache) == 0
    k64, v64, q64 = f64(k), f64(v), f64(q)
    for b in range(B):
        assert_close(out[b], oracle_out(k64[b], v64[b], q64[b], n, W), f"paged pool b={b}")


def test_validate_reports_bad_table_entry():
    """swa_validate flags live slots whose page id is outside the pool (it
    reads only the table and positions, never a page)."""
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 2, 2, 128, 64
    cache = swa.KVCache("bf16", B, H, D, W, layout="paged")
    g = torch.Generator().manual_seed(1)
    k = torch.randn((B, H, 40, D), generator=g).to(torch.bfloat16).cuda()
    swa.kv_append(cache, k, k)
    assert swa.validate(cache) == 0
    cache.block_table[1, 1] = cache.num_pages + 5   # block 1 (slots 16..31) is live
    assert swa.validate(cache) == 16
    cache.block_table[1, 3] = -1                    # block 3 (slots 48..63) is not live yet
    assert swa.validate(cache) == 16
