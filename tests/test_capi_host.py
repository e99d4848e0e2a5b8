"""Host-side checks of the C ABI: the library loads, exports every entry point
include/swa.h declares, and rejects bad arguments before launching anything
(none of these calls reaches the GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

from tests.conftest import ROOT

LIB = os.path.join(ROOT, "sliding_window_attention_ring_amd", "libswa.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libswa.so not built")


def declared_functions():
    text = open(os.path.join(ROOT, "include", "swa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def test_header_and_exports_agree():
    from sliding_window_attention_ring_amd import _capi
    decl = declared_functions()
    assert decl == set(_capi.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert decl <= exported
    L = _capi.lib()
    for name in decl:
        assert hasattr(L, name)


def desc(**kw):
    from sliding_window_attention_ring_amd._capi import SwaCacheDesc
    base = dict(kind=0, B=2, H=4, D=128, W=64, layout=0, k=0x10000, v=0x20000, pos=0x30000,
                next_position=0x40000, k_scale=0x50000, v_scale=0x60000, witness=0x70000,
                k_stage=0x80000, v_stage=0x90000, block_table=0xC0000, num_pages=8, request_id=None, layer=0,
                step_sync=0xE0000)
    base.update(kw)
    return SwaCacheDesc(**base)


def test_status_strings():
    from sliding_window_attention_ring_amd import _capi
    for code in range(-6, 1):
        assert _capi.status_string(code) and _capi.status_string(code) != "unknown status"
    assert _capi.status_string(-99) == "unknown status"


def test_argument_checks_return_codes():
    from sliding_window_attention_ring_amd._capi import lib
    L = lib()
    p = ctypes.byref
    d = desc()
    A16, ODD = ctypes.c_void_p(0xA0000), ctypes.c_void_p(0xA0004)
    ws = ctypes.c_void_p(0xB0000)
    assert L.kv_append(None, A16, A16, 1, None) == -2                       # NULL cache
    assert L.kv_append(p(desc(B=0)), A16, A16, 1, None) == -1               # B < 1
    assert L.kv_append(p(desc(layout=2)), A16, A16, 1, None) == -1              # unknown layout
    assert L.kv_append(p(desc(layout=1, W=20)), A16, A16, 1, None) == -1        # paged W % 16
    assert L.kv_append(p(desc(layout=1, num_pages=0)), A16, A16, 1, None) == -1
    assert L.kv_append(p(desc(layout=1, block_table=None)), A16, A16, 1, None) == -2
    assert L.kv_append(p(desc(layout=1, block_table=0xC0002)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(layout=1)), None, A16, 1, None) == -2         # valid: reaches the argument checks
    assert L.kv_append(p(desc(D=100)), A16, A16, 1, None) == -1             # head_dim outside {16..256}
    assert L.kv_append(p(desc(kind=7)), A16, A16, 1, None) == -4
    assert L.kv_append(p(desc(kind=2, W=20)), A16, A16, 1, None) == -1      # INT8 W % 16
    assert L.kv_append(p(desc(kind=2, D=64)), A16, A16, 1, None) == -4      # INT8 takes D = 128 only
    assert L.kv_append(p(desc(kind=2, witness=None)), A16, A16, 1, None) == -2
    assert L.kv_append(p(desc(k=0x10004)), A16, A16, 1, None) == -3         # alignment
    assert L.kv_append(p(d), ODD, A16, 1, None) == -3
    assert L.kv_append(p(d), None, A16, 1, None) == -2
    assert L.kv_append(p(d), A16, A16, -1, None) == -1
    assert L.kv_append(p(d), A16, A16, 0, None) == -1                       # T < 1
    # every descriptor field is checked on its own
    assert L.kv_append(p(desc(H=0)), A16, A16, 1, None) == -1               # H < 1
    assert L.kv_append(p(desc(W=0)), A16, A16, 1, None) == -1               # W < 1
    assert L.kv_append(p(desc(B=65536)), A16, A16, 1, None) == -1           # grid limits
    assert L.kv_append(p(desc(H=65536)), A16, A16, 1, None) == -1
    assert L.kv_append(p(desc(D=256, W=8388608)), None, A16, 1, None) == -1  # one (b, h) region reaches 4 GiB
    assert L.kv_append(p(desc(v=0x20004)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(pos=0x30002)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(next_position=0x40002)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(kind=2, k_stage=0x80004)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(kind=2, v_stage=0x90004)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(kind=2, k_scale=0x50002)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(kind=2, v_scale=0x60002)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(kind=2, witness=0x70004)), A16, A16, 1, None) == -3
    assert L.kv_truncate(p(d), A16, ctypes.c_void_p(0xA0002), None) == -3    # ok misaligned
    assert L.kv_truncate(p(d), ctypes.c_void_p(0xA0002), None, None) == -3   # cut misaligned
    need = L.swa_workspace_bytes(p(d))
    assert need > 0 and L.swa_workspace_bytes(p(desc(D=100))) == 0
    assert L.decode_attn(p(d), A16, A16, ws, need - 1, None) == -5           # small workspace
    assert L.decode_attn(p(d), ODD, A16, ws, need, None) == -3
    assert L.decode_attn(p(desc(kind=2)), A16, A16, ws, need, None) == -4    # INT8 needs the witness entry
    assert L.decode_attn_int8_witness(p(d), A16, A16, A16, None, ws, need, None) == -4
    assert L.decode_attn_int8_witness(p(desc(kind=2)), A16, A16, None, None, ws, 1 << 30, None) == -2
    i8 = desc(kind=2)
    assert L.decode_attn_int8_witness_tv(p(i8), A16, A16, A16, None, A16, 0.2, None, ws, 1 << 30, None) == -2
    assert L.decode_attn_int8_witness_tv(p(i8), A16, A16, A16, A16, A16, float("nan"), None, ws, 1 << 30,
                                         None) == -1
    assert L.decode_attn_int8_witness_tv(p(d), A16, A16, A16, A16, A16, 0.2, None, ws, 1 << 30, None) == -4
    O2 = ctypes.c_void_p(0xA0002)
    assert L.decode_attn_int8_witness_tv(p(i8), A16, A16, O2, None, None, 0.2, None, ws, 1 << 30, None) == -3
    assert L.decode_attn_int8_witness_tv(p(i8), A16, A16, A16, None, None, 0.2, O2, ws, 1 << 30, None) == -3
    assert L.decode_attn_int8_witness_tv(p(i8), A16, A16, A16, O2, None, 0.2, None, ws, 1 << 30, None) == -3
    assert L.decode_attn_int8_witness_tv(p(i8), A16, A16, A16, A16, O2, 0.2, None, ws, 1 << 30, None) == -3
    # Tier B kind: no witness needed, request ids required, delta in (0, 1]
    dz = desc(kind=3, witness=None, request_id=0xD0000)
    nz = L.swa_workspace_bytes(p(dz))
    assert nz > 0 and nz % 256 == 0  # split partials, padded to 256 bytes
    assert L.kv_append(p(dz), None, A16, 1, None) == -2
    assert L.kv_append(p(desc(kind=3, request_id=None)), A16, A16, 1, None) == -2
    assert L.kv_append(p(desc(kind=3, request_id=0xD0004)), A16, A16, 1, None) == -3
    assert L.kv_append(p(desc(kind=3, request_id=0xD0000, D=64)), A16, A16, 1, None) == -4
    dd = L.decode_attn_int8_dither
    assert dd(p(dz), A16, A16, A16, A16, A16, 0.2, 0.0, ws, nz, None) == -1        # delta = 0
    assert dd(p(dz), A16, A16, A16, A16, A16, 0.2, 1.5, ws, nz, None) == -1        # delta > 1
    assert dd(p(dz), A16, A16, A16, A16, A16, 0.2, float("nan"), ws, nz, None) == -1
    assert dd(p(dz), A16, A16, A16, A16, A16, float("nan"), 0.1, ws, nz, None) == -1
    assert dd(p(dz), A16, A16, A16, None, A16, 0.2, 0.1, ws, nz, None) == -2       # gate without tv
    assert dd(p(dz), A16, A16, None, None, None, 0.2, 0.1, ws, nz, None) == -2     # cert NULL
    assert dd(p(dz), A16, A16, A16, None, None, 0.2, 0.1, ws, nz - 1, None) == -5
    assert dd(p(i8), A16, A16, A16, None, None, 0.2, 0.1, ws, nz, None) == -4      # Tier A cache
    assert L.decode_attn_int8_witness(p(dz), A16, A16, A16, None, ws, nz, None) == -4
    assert L.decode_attn(p(dz), A16, A16, ws, nz, None) == -4
    assert L.decode_step(p(i8), A16, A16, A16, A16, ws, 1 << 30, None) == -4                  # INT8 cache
    assert L.decode_step(p(d), None, A16, A16, A16, ws, need, None) == -2
    assert L.decode_step(p(d), A16, ODD, A16, A16, ws, need, None) == -3
    assert L.decode_step(p(d), A16, A16, A16, A16, ws, need - 1, None) == -5
    st = L.decode_step_int8
    assert st(p(d), A16, A16, A16, A16, A16, None, None, 0.2, 0.1, ws, need, None) == -4     # bf16 cache
    assert st(p(i8), None, A16, A16, A16, A16, None, None, 0.2, 0.1, ws, 1 << 30, None) == -2
    assert st(p(i8), ODD, A16, A16, A16, A16, None, None, 0.2, 0.1, ws, 1 << 30, None) == -3
    assert st(p(i8), A16, A16, A16, A16, A16, None, A16, 0.2, 0.1, ws, 1 << 30, None) == -2   # gate without tv
    assert st(p(i8), A16, A16, A16, A16, A16, None, None, float("nan"), 0.1, ws, 1 << 30, None) == -1
    assert st(p(dz), A16, A16, A16, A16, A16, None, None, 0.2, 0.0, ws, nz, None) == -1       # Tier B delta
    assert st(p(dz), A16, A16, A16, A16, A16, None, None, 0.2, 0.1, ws, nz - 1, None) == -5
    assert L.swa_validate(p(d), None, None) == -2
    assert L.swa_workspace_init(None, 64, None) == -2
    assert L.swa_workspace_init(ODD, 64, None) == -3
    assert L.swa_workspace_init(A16, 0, None) == 0


def test_workspace_size_follows_split_plan():
    """Workspace = B*H*nsplit*(D+4) floats of split partials, padded to 256
    bytes, and nothing else (the fused step's counters live in the cache)."""
    from sliding_window_attention_ring_amd._capi import lib
    L = lib()
    for kw in [dict(kind=0, B=16, H=32, D=128, W=32768), dict(kind=2, B=16, H=32, D=128, W=32768),
               dict(kind=1, B=1, H=2, D=16, W=4), dict(kind=0, B=4, H=8, D=128, W=131072)]:
        d = desc(**kw)
        nb = L.swa_workspace_bytes(ctypes.byref(d))
        per = kw["B"] * kw["H"] * (kw["D"] + 4) * 4
        assert nb % 256 == 0 and nb > 0
        assert any((ns * per + 255) // 256 * 256 == nb for ns in range(1, kw["W"] + 1))


def test_every_head_dim_of_the_contract():
    """D in {16, 32, 64, 128, 256} for the bf16 and fp32 kinds; the INT8 kinds
    take 128 only (SWA_EUNSUPPORTED otherwise); any other D is SWA_EINVAL."""
    from sliding_window_attention_ring_amd._capi import lib
    L = lib()
    A16 = ctypes.c_void_p(0xA0000)
    for kind in range(4):
        for D in (16, 32, 64, 128, 256):
            extra = dict(request_id=0xD0000) if kind == 3 else {}
            d = desc(kind=kind, D=D, **extra)
            want = -2 if (kind < 2 or D == 128) else -4   # valid: kv_append reaches its NULL k_new check
            assert L.kv_append(ctypes.byref(d), None, A16, 1, None) == want, (kind, D)
            assert (L.swa_workspace_bytes(ctypes.byref(d)) > 0) == (want == -2)
        for D in (0, 8, 48, 96, 512):
            assert L.kv_append(ctypes.byref(desc(kind=kind, D=D)), None, A16, 1, None) == -1


def test_fused_steps_need_the_completion_counters():
    from sliding_window_attention_ring_amd._capi import lib
    L = lib()
    p = ctypes.byref
    A16, ws = ctypes.c_void_p(0xA0000), ctypes.c_void_p(0xB0000)
    d, i8 = desc(step_sync=None), desc(kind=2, step_sync=None)
    assert L.decode_step(p(d), A16, A16, A16, A16, ws, 1 << 30, None) == -2
    assert L.decode_step_int8(p(i8), A16, A16, A16, A16, A16, None, None, 0.2, 0.1, ws, 1 << 30, None) == -2
    assert L.kv_append(p(d), None, A16, 1, None) == -2                   # the other calls do not need them
    assert L.kv_append(p(desc(step_sync=0xE0002)), None, A16, 1, None) == -3   # misaligned counters


def test_static_scratch_step_checks_its_arguments_before_any_hip_call():
    """decode_step_int8_static rejects bad arguments exactly as
    decode_step_int8 does, and an oversized shape, before it touches HIP
    (these calls run on a host without a GPU)."""
    from sliding_window_attention_ring_amd._capi import lib
    L = lib()
    p = ctypes.byref
    A16, ODD = ctypes.c_void_p(0xA0000), ctypes.c_void_p(0xA0004)
    st = L.decode_step_int8_static
    i8, dz = desc(kind=2), desc(kind=3, witness=None, request_id=0xD0000)
    assert st(None, A16, A16, A16, A16, A16, None, None, 0.2, 0.1, None) == -2
    assert st(p(desc()), A16, A16, A16, A16, A16, None, None, 0.2, 0.1, None) == -4       # bf16 cache
    assert st(p(i8), None, A16, A16, A16, A16, None, None, 0.2, 0.1, None) == -2
    assert st(p(i8), A16, A16, A16, A16, None, None, None, 0.2, 0.1, None) == -2          # cmax NULL
    assert st(p(desc(kind=2, step_sync=None)), A16, A16, A16, A16, A16, None, None, 0.2, 0.1, None) == -2
    assert st(p(i8), ODD, A16, A16, A16, A16, None, None, 0.2, 0.1, None) == -3
    assert st(p(i8), A16, A16, A16, A16, A16, None, A16, 0.2, 0.1, None) == -2            # gate without tv
    assert st(p(i8), A16, A16, A16, A16, A16, None, None, float("nan"), 0.1, None) == -1
    assert st(p(dz), A16, A16, A16, A16, A16, None, None, 0.2, 0.0, None) == -1          # Tier B delta
    big = desc(kind=2, B=65535, H=2, W=16)                                                # 69 MB of partials
    assert L.swa_workspace_bytes(p(big)) > 16 << 20
    assert st(p(big), A16, A16, A16, A16, A16, None, None, 0.2, 0.1, None) == -5
