"""The bandwidth target, as a GPU test: the fused decode step at 32768
context (B=16, H=32, D=128) must move its algorithmic bytes at >= 70% of
MI355X's 8 TB/s HBM peak -- the INT8 cache with the witness bound (the
headline), the dithered INT8 cache with its certificate, and the bf16 cache.

Bytes of one INT8 step (the storage format of page "WitCert", section
频带酉性与双层证书: 16 bands of fp16 per token and head; section SGLang
生产级落地: one fp32 scale per block and tensor): 288.5 B per visible
quantized token-head (codes 2 x 128, witness 32, scales 0.5; 256.5 B
without the witness), 512 B per staged token-head (bf16 K and V rows), the
query, the output and the bound, plus the append (the new rows read and
written).  A bf16 step reads 512 B per visible token-head.  The cache is
filled with valid values directly (random codes, fixed block scales and
band norms, a full window) instead of a prefill: the step reads the same
bytes whatever they hold.  Warm-up steps run first, past the clock
transient that follows the idle set-up.
"""

import pytest
import torch

from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

PEAK_BYTES_PER_S = 8.0e12
TARGET = 0.70


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def step_bytes(kind, B, H, D, W, n_after):
    append = B * H * 2 * D * 2 * 2
    q_out = B * H * (D * 2 + D * 4)
    if kind == "bf16":
        return B * H * min(W, n_after) * 2 * D * 2 + q_out + append
    staged = n_after % 16
    quant = min(W, n_after) - staged
    wit = 2 * D // 8 if kind == "int8" else 0
    return B * H * (quant * (2 * D + wit + 2 * 4 / 16) + staged * 2 * D * 2) + q_out + B * H * 4 + append


@pytest.mark.parametrize("kind", ["int8", "int8_dither", "bf16"])
def test_decode_step_at_32k_meets_the_bandwidth_target(kind):
    import sliding_window_attention_ring_amd as swa
    B, H, D, W = 16, 32, 128, 32768
    warmup, steps = 80, 20
    say("bandwidth target:", kind, "step", B, H, D, W)
    c = swa.KVCache(kind, B, H, D, W)
    g = torch.Generator(device="cuda").manual_seed(3)
    if kind == "bf16":
        c.k.copy_(torch.randn(c.k.shape, generator=g, device="cuda").to(torch.bfloat16))
        c.v.copy_(torch.randn(c.v.shape, generator=g, device="cuda").to(torch.bfloat16))
    else:
        c.k.copy_(torch.randint(-127, 128, c.k.shape, generator=g, device="cuda", dtype=torch.int8))
        c.v.copy_(torch.randint(-127, 128, c.v.shape, generator=g, device="cuda", dtype=torch.int8))
        c.k_scale.fill_(0.02)
        c.v_scale.fill_(0.02)
        if kind == "int8":
            c.witness.fill_(1e-3)
        c.k_stage.copy_(torch.randn(c.k_stage.shape, generator=g, device="cuda").to(torch.bfloat16))
        c.v_stage.copy_(torch.randn(c.v_stage.shape, generator=g, device="cuda").to(torch.bfloat16))
    n0 = 2 * W + 5
    c.next_position.fill_(n0)
    kn = torch.randn((B, H, 1, D), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((B, H, 1, D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, H, D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    cmax = torch.empty((B, H), dtype=torch.float32, device="cuda")
    ws = c.workspace()

    def step():
        if kind == "bf16":
            swa.decode_step(c, kn, vn, q, out=out, ws=ws)
        else:
            swa.decode_step_int8(c, kn, vn, q, delta=1e-6, out=out, cmax=cmax, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) / 1e3
    total = sum(step_bytes(kind, B, H, D, W, n0 + warmup + i + 1) for i in range(steps))
    rate = total / sec
    say(f"{kind}: {sec / steps * 1e3:.4f} ms per step, {rate / 1e12:.3f} TB/s, {rate / PEAK_BYTES_PER_S:.1%} of peak")
    assert int(c.next_position[0]) == n0 + warmup + steps
    assert torch.isfinite(out).all() and (kind == "bf16" or torch.isfinite(cmax).all())
    assert rate >= TARGET * PEAK_BYTES_PER_S, f"{rate / 1e12:.3f} TB/s is below 70% of 8 TB/s"
