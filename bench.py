"""Decode-step benchmark on one MI355X.

A step is one pass of the decode hot path over the whole batch: one token
per sequence is appended and one query per sequence attends to the cache.
By default a step is one call of the fused entry point (``decode_step_int8``
for the INT8 workloads, with the witness bound, or with the certificate, TV
bound and gate for the dithered one; ``decode_step`` otherwise), which
appends and attends in one launch.  When a (b, h) has several splits, a
merge launch follows for the INT8 kinds; the row kinds merge them in the
step kernel (up to 63 heads).  ``--no-fuse`` times ``kv_append`` followed by the separate
decode call instead.  The default workload is the INT8 cache with the
witness bound at 32768 context (B=16, H=32, D=128), prefilled with 32768
rotary keys.

A workload whose step reads under 2 GiB (the ring of 4096, the ragged
batch, the one-GPU shard shapes, the tiny window) would find part of its
bytes in the 256 MB MALL left by the step before; its calls rotate over 3-8
identical instances of the cache instead, so each step reads its K/V from
HBM and one pair of events still spans all timed calls.

Prints ONE JSON line on stdout.  ``value`` is the whole step's algorithmic
HBM bytes per second (GB/s); ``roofline`` reports the timed call alone,
timed with HIP events on its launch stream; ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload.

Before the warmup steps, decode-only calls (which change no cache state) run
for --settle-ms (50 ms by default), so that the timed steps do not start in
the clock transient that follows the idle setup; their count is reported in
``config.settle``.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 20]
       [--workload NAME] [--no-cpu-baseline] [--no-fuse]
       [--rotate auto|on|off] [--settle-ms 50] [--calibrate-copy]
"""

from __future__ import annotations

import argparse
import hashlib
from dataclasses import replace
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn achieved HBM GB/s (% of peak) + tokens·heads/s at 32k ctx"
PEAK_GBS = 8000.0  # MI355X HBM3E peak
# Per-query failure budget of the dithered INT8 certificate (one (b, h)).
DITHER_DELTA = 1e-6
CSRC = os.path.join(ROOT, "sliding_window_attention_ring_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kind: str) -> str:
    """Hash of the decode kernel's sources with line comments and blank lines
    left out, so that a counter summary stays valid across comment edits and
    lapses with any change to the code."""
    files = (["swa_device.h", "swa_commit.h", "swa_decode_int8.hip"] if kind.startswith("int8")
             else ["swa_device.h", "swa_decode.hip"])
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def read_traffic(workload: str, kind: str):
    """HBM bytes per decode launch from the committed counter summary, or None
    if there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"{workload}_decode_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith("#"):
            a, b = ln.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash(kind):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def step_bytes(wl, n_after):
    """Algorithmic HBM bytes of one step whose append brings next_position to
    n_after (an int, or one int per sequence): (decode bytes, append bytes,
    visible tokens summed over sequences, per head)."""
    if not isinstance(n_after, int):
        parts = [step_bytes(replace(wl, B=1), int(n)) for n in n_after]
        return tuple(sum(p[i] for p in parts) for i in range(3))
    BH, D = wl.B * wl.H, wl.D
    vis = min(wl.W, n_after) * wl.B
    q_out = BH * D * 2 + BH * D * 4
    if wl.kind in ("int8", "int8_dither"):
        wit = 2 * D // 8 if wl.kind == "int8" else 0   # fp16 band norms per token-head (Tier A only)
        outs = 4 if wl.kind == "int8" else 12           # cmax, or cert + tv + gate
        staged = n_after % 16
        quant = min(wl.W, n_after) - staged
        dec = BH * (quant * (2 * D + wit + 2 * 4 / 16) + staged * 2 * D * 2) + q_out + BH * outs
        app = BH * 2 * D * 2 * 2  # read the new rows, write them to staging
        if n_after % 16 == 0:     # a block completes: read 16 staged rows, write codes/witness/scales
            app += BH * 16 * (2 * D * 2 + 2 * D + wit) + BH * 2 * 4
    else:
        esz = 4 if wl.kind == "fp32" else 2
        dec = BH * min(wl.W, n_after) * 2 * D * esz + (BH * D * esz + BH * D * 4)
        app = BH * 2 * D * esz * 2 + wl.B * 4
    return dec, app, vis


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Threads for the all-cores oracle run: OMP_NUM_THREADS if set (the
    box's CPU share), else the affinity core count."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    return int(env) if env.isdigit() and int(env) > 0 else len(os.sched_getaffinity(0))


def cpu_baseline(wl, k_all, v_all, q, ns, budget_s: float = 12.0, threads: int = 1):
    """Time the oracle (as it stands) on a sample of (b, h) pairs of the same
    workload, sequence b at next_position ns[b], with ``threads`` BLAS/OpenMP
    threads; GB/s of algorithmic bytes.  ``q`` is the query [B, H, D]."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention, bits, dither as odither, int8 as oint8
    from workloads import gen

    # A seeded sample of (b, h) pairs, as many as fit in 2 GiB of float64
    # inputs (at most 256), widened once outside the timed oracle calls; the
    # calls then cycle over the sample until the time budget is spent.
    rng = np.random.default_rng(2026)
    pair_bytes = 2 * min(wl.W, max(int(n) for n in ns)) * wl.D * 8
    n_pairs = max(1, min(256, (2 << 30) // pair_bytes))
    pairs = [(int(rng.integers(wl.B)), int(rng.integers(wl.H))) for _ in range(n_pairs)]
    qb = gen.to_bits(q)
    one = replace(wl, B=1)
    held = {}
    for b, h in pairs:
        if (b, h) not in held:
            n = int(ns[b])
            held[(b, h)] = (bits.to_f64(gen.to_bits(k_all[b, h, :n])), bits.to_f64(gen.to_bits(v_all[b, h, :n])))
    done, t_used, nbytes, kv, t_log = 0, 0.0, 0.0, 0, time.time()
    with threadpool_limits(limits=threads):
        for i in range(256 * 1000):
            b, h = pairs[i % len(pairs)]
            n = int(ns[b])
            kk, vv = held[(b, h)]
            qq = bits.to_f64(qb[b, h])
            t0 = time.perf_counter()
            if wl.kind == "int8":
                oint8.int8_decode(qq, kk, vv, n, wl.W)
            elif wl.kind == "int8_dither":
                odither.int8_dither_decode(qq, kk, vv, n, wl.W, b, 0, h, DITHER_DELTA)
            else:
                attention.masked_attention(qq, np.arange(n), kk, vv, n - 1, wl.W)
            t_used += time.perf_counter() - t0
            done += 1
            nbytes += step_bytes(one, n)[0] / wl.H
            kv += min(wl.W, n)
            if time.time() - t_log > 10:
                log(f"[bench] oracle: {done} calls, {t_used:.1f} s")
                t_log = time.time()
            if t_used >= budget_s:
                break
    lo, hi = min(min(wl.W, int(n)) for n in ns), max(min(wl.W, int(n)) for n in ns)
    ctx = f"context {lo}" if lo == hi else f"contexts {lo}..{hi}"
    return {
        "value": nbytes / t_used / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} oracle calls on {min(done, len(held))} sampled (b,h) pairs of {wl.name} at {ctx}, "
                  f"float64 NumPy, {threads} thread(s) of "
                  f"{len(os.sched_getaffinity(0))} affinity cores ({cpu_model()}), {t_used:.1f} s "
                  f"({kv / t_used:.3g} KV-token-heads/s)",
        "kv_token_heads_per_s": kv / t_used,
    }


def device_info(torch) -> dict:
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / (1 << 30), 1)}


def main():
    from workloads import ALL, INT8_32K

    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=INT8_32K.name, choices=sorted(ALL))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fuse", action="store_true",
                    help="time kv_append + the decode call instead of the one decode_step / decode_step_int8 call")
    ap.add_argument("--rotate", choices=("auto", "on", "off"), default="auto",
                    help="rotate the calls over 3-8 instances of the cache, so that no K/V bytes of a step are "
                         "served from the 256 MB MALL or L2; auto = on when a step reads under 2 GiB")
    ap.add_argument("--settle-ms", type=float, default=50.0,
                    help="before the warmup steps, run decode-only calls (no cache state changes) for this many "
                         "milliseconds, so that the timed steps do not start in the clock transient that follows "
                         "the idle setup; 0 disables")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode step needs no exchange when heads or sequences are split over GPUs.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sliding_window_attention_ring_amd as swa
    from workloads import gen

    wl = ALL[args.workload]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_steps = args.warmup + args.steps
    prefill = wl.prefill or wl.W
    lens = gen.ragged_lengths(wl) if wl.ragged else None  # per-sequence prefill lengths
    # Cold steps: a step that reads under 2 GiB would find part of its K/V
    # bytes in the 256 MB MALL (and L2) left by the step before.  The calls
    # then rotate over several instances of the cache, so that between two
    # steps on one instance the others read at least 2 GiB; no flush kernel
    # and no per-call event marker enters the timed region.
    est = step_bytes(wl, prefill + 1 if lens is None else [int(n) + 1 for n in lens])[0]
    cold = args.rotate == "on" or (args.rotate == "auto" and est < 2 * (1 << 30))
    n_inst = min(8, max(3, -(-(2 << 30) // int(est)) + 1)) if cold else 1
    per_inst = -(-n_steps // n_inst)  # steps each instance takes
    total = prefill + per_inst
    log(f"[bench] workload {wl.name}: B={wl.B} H={wl.H} D={wl.D} W={wl.W} prefill={prefill} "
        f"steps={args.steps} warmup={args.warmup} cache instances={n_inst}")

    t0 = time.time()
    k_all = gen.tokens(wl, "k", total, device=dev)
    v_all = gen.tokens(wl, "v", total, device=dev)
    caches = []
    for _ in range(n_inst):
        cache = swa.KVCache(wl.kind, wl.B, wl.H, wl.D, wl.W, device=dev, layout=wl.layout)
        if lens is not None:
            for b, n in enumerate(lens):
                swa.kv_append(cache.seq_view(b), k_all[b:b + 1, :, :n].contiguous(),
                              v_all[b:b + 1, :, :n].contiguous())
        else:
            chunk = wl.prefill_chunk or prefill
            for c0 in range(0, prefill, chunk):
                c1 = min(prefill, c0 + chunk)
                swa.kv_append(cache, k_all[:, :, c0:c1].contiguous(), v_all[:, :, c0:c1].contiguous())
        caches.append((cache, cache.workspace()))
    ks = [k_all[:, :, p:p + 1].contiguous() for p in range(prefill, total)]
    vs = [v_all[:, :, p:p + 1].contiguous() for p in range(prefill, total)]
    qs = [gen.query(wl, p, device=dev) for p in range(prefill, total)]
    out = torch.empty((wl.B, wl.H, wl.D), dtype=torch.float32, device=dev)
    cmax = torch.empty((wl.B, wl.H), dtype=torch.float32, device=dev)
    tv = torch.empty((wl.B, wl.H), dtype=torch.float32, device=dev)
    gate = torch.empty((wl.B, wl.H), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.time() - t0:.1f} s")

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # Call c goes to instance c mod n_inst, as that instance's step c div n_inst.
    # One call per step: kv_append of the token and the decode, fused into
    # one launch (INT8 kinds: plus the merge launch when a (b, h) has several
    # splits).
    fuse = not args.no_fuse
    dither = wl.kind == "int8_dither"

    def decode(cache, ws, q):
        if wl.kind == "int8":
            swa.decode_attn_int8_witness(cache, q, out=out, cmax=cmax, ws=ws)
        elif wl.kind == "int8_dither":
            swa.decode_attn_int8_dither(cache, q, delta=DITHER_DELTA, out=out, cert=cmax, tv=tv, gate=gate, ws=ws)
        else:
            swa.decode_attn(cache, q, out=out, ws=ws)

    def fused(c):
        cache, ws = caches[c % n_inst]
        i = c // n_inst
        if wl.kind in ("int8", "int8_dither"):
            swa.decode_step_int8(cache, ks[i], vs[i], qs[i], tau=0.2, delta=DITHER_DELTA, out=out, cmax=cmax,
                                 tv=tv if dither else None, gate=gate if dither else None, ws=ws)
        else:
            swa.decode_step(cache, ks[i], vs[i], qs[i], out=out, ws=ws)

    def append(c):
        cache, _ = caches[c % n_inst]
        swa.kv_append(cache, ks[c // n_inst], vs[c // n_inst])

    # Settle: the GPU idled while the host prepared the inputs, and the first
    # ~20 steps after such a pause run up to 10% slower as the clock settles
    # (kernel traces show it on every part).  A serving loop decodes back to
    # back, so decode-only calls, which read the same bytes and change no
    # cache state, run for --settle-ms before the warmup steps.
    settle_calls = 0
    if args.settle_ms > 0:
        t_settle = time.perf_counter()
        while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
            for _ in range(4):
                decode(*caches[settle_calls % n_inst], qs[0])
                settle_calls += 1
            torch.cuda.synchronize()

    for c in range(args.warmup):
        if fuse:
            fused(c)
        else:
            append(c)
            decode(*caches[c % n_inst], qs[c // n_inst])
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    dec_bytes = app_bytes = vis_tokens = 0.0
    positions = []
    for c in range(args.warmup, n_steps):
        done = c // n_inst + 1  # the instance's steps after this call
        positions.append(prefill + done - 1)
        d, a, vis = step_bytes(wl, prefill + done if lens is None else [int(n) + done for n in lens])
        dec_bytes, app_bytes, vis_tokens = dec_bytes + d, app_bytes + a, vis_tokens + vis
    # An event pair around each decode call only where the timed call must be
    # told apart from other work in the stream (the append of --no-fuse):
    # each event marker costs the stream about 4 us.  Otherwise one pair of
    # events spans the K calls, and a call's time is their average, launch
    # gaps included.
    per_call = not fuse
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
    span = tuple(torch.cuda.Event(enable_timing=True) for _ in range(2))
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if not per_call:
        span[0].record(stream)
    for i, c in enumerate(range(args.warmup, n_steps)):
        if fuse:
            fused(c)
        else:
            append(c)
            evs[i][0].record(stream)
            decode(*caches[c % n_inst], qs[c // n_inst])
            evs[i][1].record(stream)
    if not per_call:
        span[1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    if per_call:
        dec_ms = sorted(e1.elapsed_time(e2) for e1, e2 in evs)
        kern_ms = sum(dec_ms) / args.steps
        kern_median = dec_ms[args.steps // 2] if args.steps % 2 else 0.5 * (dec_ms[args.steps // 2 - 1] + dec_ms[args.steps // 2])
    else:
        kern_ms = kern_median = span[0].elapsed_time(span[1]) / args.steps

    ms_per_step = elapsed * 1e3 / args.steps
    value = (dec_bytes + app_bytes) / elapsed / 1e9
    # the timed call: the decode, or with fuse the whole step (append included)
    timed_bytes = (dec_bytes + app_bytes) if fuse else dec_bytes
    achieved = (timed_bytes / args.steps) / (kern_ms * 1e-3) / 1e9
    BH = wl.B * wl.H
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "head_dim": wl.D, "window": wl.W,
                   "context": min(wl.W, prefill) if lens is None else [int(n) for n in lens],
                   "kv_dtype": wl.kind, "layout": wl.layout, "cache_instances": n_inst,
                   "settle": {"ms": args.settle_ms, "decode_only_calls": settle_calls},
                   "positions": [min(positions), max(positions)],
                   "step": ("decode_step (kv_append of one token + decode_attn, one call)" if wl.kind in ("bf16", "fp32")
                            else "decode_step_int8 (kv_append of one token + the decode, one call; "
                            + ("cert, tv, gate, delta=%g)" % DITHER_DELTA if dither else "witness bound)")) if fuse
                   else "kv_append(T=1) + " + {"int8": "decode_attn_int8_witness",
                                               "int8_dither": "decode_attn_int8_dither (cert, tv, gate; "
                                                              f"delta={DITHER_DELTA})"}.get(wl.kind, "decode_attn")},
        "pct_of_peak": round(100 * value / PEAK_GBS, 2),
        "kv_token_heads_per_s": vis_tokens * wl.H / elapsed,
        "query_token_heads_per_s": BH * args.steps / elapsed,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": read_traffic(wl.name, wl.kind),
            "kernel": (("decode_step_int8_kernel (the step call; plus the merge kernel when a (b, h) has several "
                        "splits)" if wl.kind.startswith("int8") else
                        "decode_step_rows_kernel (the step call; several splits per (b, h) merge in it up to 63 "
                        "heads, else in the merge kernel)") if fuse else
                       "decode_int8_kernel" if wl.kind.startswith("int8") else "decode_kernel"),
            "kernel_ms": round(kern_ms, 4),
            "kernel_ms_median": round(kern_median, 4),
            "timing": ("HIP event pair around each timed decode call on its stream" if per_call else
                       "HIP event pair around the K timed calls on their stream (average per call, launch gaps "
                       "included)"),
            "algorithmic_bytes_per_launch": timed_bytes / args.steps,
        },
        "cpu_baseline": None,
        "cpu_baseline_all_cores": None,
        "device": device_info(torch),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample (1 thread, then all cores) ...")
        ns = [prefill] * wl.B if lens is None else [int(n) for n in lens]
        q = gen.query(wl, prefill - 1)
        result["cpu_baseline"] = cpu_baseline(wl, k_all, v_all, q, ns)
        result["cpu_baseline_all_cores"] = cpu_baseline(wl, k_all, v_all, q, ns, budget_s=8.0,
                                                        threads=host_threads())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
