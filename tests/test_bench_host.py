"""Host logic of bench.py (no GPU): the algorithmic bytes behind the
roofline figure, the refusal of more than one GPU, and the rule that a
counter summary taken on another kernel source is not reported.

The per-unit byte figures are the method's storage: bf16 K and V rows are
2*D*2 = 512 bytes per token and head; an INT8 token-head reads 128 + 128
code bytes, 16 fp16 band norms (32 bytes) and 2 fp32 block scales shared by
16 tokens (0.5 bytes); the dithered INT8 kind stores no band norms.  The
query (bf16) and the output (fp32) are read and written once per (b, h).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def _io(wl, extra_out_bytes):
    bh = wl.B * wl.H
    return bh * wl.D * 2 + bh * wl.D * 4 + bh * extra_out_bytes


@pytest.mark.parametrize("name,n,kv_bytes,outs", [
    # 16*32 token-heads of 32768 tokens at 288.5 B
    ("int8-witness-ctx32768", 32768, 4_840_226_816, 4),
    # the same without band norms: 256.5 B; cert, tv and gate per (b, h)
    ("int8-dither-ctx32768", 32768, 4_303_355_904, 12),
    ("bf16-ctx32768", 32768, 8_589_934_592, 0),
    ("long-ctx-131072-bf16", 131072, 2_147_483_648, 0),
    # the window holds 4096 of the 8193 positions
    ("ring-w4096-pos8192-bf16", 8193, 1_073_741_824, 0),
    # one GPU's 16384 of the 131072 slots
    ("long-ctx-131072-bf16-ctx-shard-1of8", 16384, 268_435_456, 0),
])
def test_decode_bytes_per_step(name, n, kv_bytes, outs):
    wl = workloads.ALL[name]
    dec, _, vis = bench.step_bytes(wl, n)
    assert dec == pytest.approx(kv_bytes + _io(wl, outs), rel=0, abs=1e-6)
    assert vis == min(wl.W, n) * wl.B


def test_int8_staged_tokens_are_read_as_bf16():
    """Five tokens past a block boundary sit in the bf16 staging rows
    (512 B per token-head); the other 32763 of the window are codes."""
    wl = workloads.ALL["int8-witness-ctx32768"]
    bh = wl.B * wl.H
    dec, app, _ = bench.step_bytes(wl, 32768 + 5)
    assert dec == pytest.approx(bh * (32763 * 288.5 + 5 * 512) + _io(wl, 4), abs=1e-6)
    # an append that does not complete a block reads the new rows and writes them to staging
    assert app == bh * 2 * wl.D * 2 * 2


def test_int8_block_commit_bytes():
    """The append that completes a block also reads the 16 staged rows and
    writes their codes, band norms and two scales."""
    wl = workloads.ALL["int8-witness-ctx32768"]
    bh = wl.B * wl.H
    _, app, _ = bench.step_bytes(wl, 32768 + 16)
    assert app == bh * 2 * wl.D * 2 * 2 + bh * 16 * (2 * wl.D * 2 + 2 * wl.D + 32) + bh * 2 * 4


def test_ragged_bytes_sum_over_sequences():
    wl = workloads.ALL["full-cache-ragged-4096-bf16"]
    lens = [1024, 4096, 2000, 5000, 1, 3000, 4095, 2048]
    dec, _, vis = bench.step_bytes(wl, lens)
    kv = sum(min(wl.W, n) for n in lens) * wl.H * 512
    assert dec == pytest.approx(kv + _io(wl, 0), abs=1e-6)
    assert vis == sum(min(wl.W, n) for n in lens)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_from_another_kernel_source_is_not_reported(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    name = "int8-witness-ctx32768"
    path = tmp_path / f"{name}_decode_traffic.txt"
    assert bench.read_traffic(name, "int8") is None  # no summary
    path.write_text("# header\nhbm_bytes_per_launch: 123456\nkernel_source_sha: 0000000000000000\n")
    assert bench.read_traffic(name, "int8") is None  # stale
    path.write_text(f"hbm_bytes_per_launch: 123456\nkernel_source_sha: {bench.kernel_source_hash('int8')}\n")
    assert bench.read_traffic(name, "int8") == 123456.0
    # the bf16 kernels hash other files
    assert bench.kernel_source_hash("bf16") != bench.kernel_source_hash("int8")


def test_kernel_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    """A comment edit keeps a counter summary valid; a code edit retires it."""
    import shutil
    for f in ("swa_device.h", "swa_decode.hip"):
        shutil.copy(os.path.join(bench.CSRC, f), tmp_path / f)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.kernel_source_hash("bf16")
    src = tmp_path / "swa_decode.hip"
    text = src.read_text()
    src.write_text("// a new comment line\n\n" + text.replace("namespace swa {", "namespace swa {  // trailing", 1))
    assert bench.kernel_source_hash("bf16") == h0
    src.write_text(text.replace("kNegBig = -1e30f", "kNegBig = -1e29f", 1))
    assert bench.kernel_source_hash("bf16") != h0


def test_cpu_baseline_times_ragged_lengths():
    """The oracle leg of the bench runs on a ragged workload too: each sampled
    pair is timed at its own sequence's length, and its bytes follow it."""
    import torch
    from dataclasses import replace
    from workloads import gen
    wl = replace(workloads.ALL["full-cache-ragged-4096-bf16"], B=3, H=2, W=64)
    ns = [10, 64, 100]
    k = gen.tokens(wl, "k", 100)
    v = gen.tokens(wl, "v", 100)
    q = gen.query(wl, 0)
    r = bench.cpu_baseline(wl, k, v, q, ns, budget_s=0.05)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    assert "contexts 10..64" in r["sample"]
    assert r["kv_token_heads_per_s"] > 0
    assert isinstance(k, torch.Tensor)
