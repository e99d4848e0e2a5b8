"""Python binding of the C ABI: torch tensors in, device pointers out.

torch provides device memory and the current HIP stream; every step of the
decode path runs in the HIP kernels of libswa.so.  The functions keep the C
names (``kv_append``, ``decode_attn``, ``decode_attn_int8_witness``, ...) and
only check and marshal their arguments.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _capi
from ._capi import KIND, LAYOUT, SwaCacheDesc, check, lib

_INPUT_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32, "int8": torch.bfloat16,
                "int8_dither": torch.bfloat16}
_STORE_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32, "int8": torch.int8, "int8_dither": torch.int8}


def _stream(stream=None) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, shape, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class KVCache:
    """Device tensors of one sliding-window cache and its descriptor.

    kind: "bf16" | "fp32" | "int8" | "int8_dither"; B sequences, H heads,
    head_dim D, window W.  "int8_dither" is INT8 with subtractive dither and
    no witness; its ``request_id`` [B] (int64 bits of the uint64 ids,
    default 0..B-1) and ``layer`` key the dither stream.
    layout "ring": ``k``, ``v`` are [B, H, W, D] (INT8: ``k_scale``/``v_scale``
    [B, H, W/16], ``witness`` [B, H, W, D/8] fp16).  layout "paged": they are
    pools of ``num_pages`` 16-token pages ([P, H, 16, D], [P, H], [P, H, 16,
    D/8]) and ``block_table`` [B, W/16] int32 names the page of each ring
    block; by default every sequence gets W/16 distinct pages in a seeded
    shuffled order.  Per-sequence tensors: ``pos`` [B, W], ``next_position``
    [B], ``step_sync`` [B, 64] (the fused step's completion counters, zero
    between calls) and, for INT8, ``k_stage``/``v_stage`` [B, H, 16, D].
    """

    def __init__(self, kind: str, B: int, H: int, D: int, W: int, device="cuda", layout: str = "ring",
                 num_pages: Optional[int] = None, block_table: Optional[torch.Tensor] = None,
                 request_id: Optional[torch.Tensor] = None, layer: int = 0):
        if kind not in KIND:
            raise ValueError(f"kind must be one of {sorted(KIND)}")
        if layout not in LAYOUT:
            raise ValueError(f"layout must be one of {sorted(LAYOUT)}")
        self.kind, self.B, self.H, self.D, self.W, self.layout = kind, B, H, D, W, layout
        dev = torch.device(device)
        if dev.type != "cuda":  # the kernels take device pointers: never hand them host memory
            raise ValueError(f"a KVCache lives in GPU memory: device must be a GPU device, got {dev}")
        paged = layout == "paged"
        if paged:
            if W % 16:
                raise ValueError("a paged cache needs W % 16 == 0")
            if block_table is not None and (not isinstance(block_table, torch.Tensor)
                                            or tuple(block_table.shape) != (B, W // 16)):
                # the kernels index the table as [B][W/16]: a smaller one would be read past its end
                raise ValueError(f"block_table must be a tensor of shape [B, W/16] = [{B}, {W // 16}]")
            self.num_pages = B * (W // 16) if num_pages is None else int(num_pages)
            rows = (self.num_pages, H, 16)
        else:
            self.num_pages = 0
            rows = (B, H, W)
        self.k = torch.empty(rows + (D,), dtype=_STORE_DTYPE[kind], device=dev)
        self.v = torch.empty_like(self.k)
        self.pos = torch.empty((B, W), dtype=torch.int32, device=dev)
        self.next_position = torch.empty((B,), dtype=torch.int32, device=dev)
        self.step_sync = torch.empty((B, 64), dtype=torch.int32, device=dev)
        self.k_scale = self.v_scale = self.witness = self.k_stage = self.v_stage = None
        if kind in ("int8", "int8_dither"):
            scales = (self.num_pages, H) if paged else (B, H, W // 16)
            self.k_scale = torch.empty(scales, dtype=torch.float32, device=dev)
            self.v_scale = torch.empty_like(self.k_scale)
            if kind == "int8":
                self.witness = torch.empty(rows + (D // 8,), dtype=torch.float16, device=dev)
            self.k_stage = torch.empty((B, H, 16, D), dtype=torch.bfloat16, device=dev)
            self.v_stage = torch.empty_like(self.k_stage)
        self.request_id, self.layer = None, int(layer)
        if kind == "int8_dither":
            if request_id is None:
                request_id = torch.arange(B, dtype=torch.int64)
            if tuple(request_id.shape) != (B,) or request_id.dtype != torch.int64:
                raise ValueError("request_id must be an int64 tensor of shape [B] (the uint64 bits)")
            self.request_id = request_id.to(dev).contiguous()
        self.block_table = None
        if paged:
            if block_table is None:
                if self.num_pages < B * (W // 16):
                    raise ValueError("pass a block_table when the pool has fewer than B*W/16 pages")
                g = torch.Generator().manual_seed(B * 1000003 + W)
                block_table = torch.randperm(self.num_pages, generator=g)[: B * (W // 16)].reshape(B, W // 16)
            self.block_table = block_table.to(device=dev, dtype=torch.int32).contiguous()
        self.desc = self._make_desc()
        self._ws = None
        cache_reset(self)

    def _make_desc(self, b: Optional[int] = None) -> SwaCacheDesc:
        paged = self.layout == "paged"

        def per_seq(t):  # tensors indexed by sequence
            if t is None:
                return None
            return t.data_ptr() if b is None else t[b].data_ptr()

        def pool(t):  # row storage: per sequence in a ring, shared in a paged pool
            if t is None:
                return None
            return t.data_ptr() if (paged or b is None) else t[b].data_ptr()

        return SwaCacheDesc(KIND[self.kind], self.B if b is None else 1, self.H, self.D, self.W,
                            LAYOUT[self.layout], pool(self.k), pool(self.v), per_seq(self.pos),
                            per_seq(self.next_position), pool(self.k_scale), pool(self.v_scale),
                            pool(self.witness), per_seq(self.k_stage), per_seq(self.v_stage),
                            per_seq(self.block_table), self.num_pages, per_seq(self.request_id),
                            self.layer & 0xFFFFFFFF, per_seq(self.step_sync))

    def seq_view(self, b: int) -> "SeqView":
        """Descriptor of sequence ``b`` alone (B = 1), for ragged appends."""
        return SeqView(self, b)

    @property
    def input_dtype(self) -> torch.dtype:
        return _INPUT_DTYPE[self.kind]

    def workspace(self) -> torch.Tensor:
        """The decode workspace of this cache (split partials), allocated once."""
        if self._ws is None:
            nbytes = workspace_bytes(self)
            self._ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.k.device)
        return self._ws


class SeqView:
    """One sequence of a KVCache as a B = 1 cache (shares the storage)."""

    def __init__(self, cache: KVCache, b: int):
        if not 0 <= b < cache.B:
            raise IndexError(b)
        self.parent, self.b = cache, b
        self.kind, self.B, self.H, self.D, self.W = cache.kind, 1, cache.H, cache.D, cache.W
        self.k = cache.k
        self.desc = cache._make_desc(b)

    @property
    def input_dtype(self) -> torch.dtype:
        return self.parent.input_dtype


def cache_reset(cache, stream=None) -> None:
    """``swa_cache_reset``: next_position = 0, every slot empty."""
    check(lib().swa_cache_reset(ctypes.byref(cache.desc), _stream(stream)), "swa_cache_reset")


def kv_append(cache, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """``kv_append``: append ``k_new``, ``v_new`` of shape [B, H, T, D]."""
    T = k_new.shape[2] if k_new.dim() == 4 else -1
    shape = (cache.B, cache.H, T, cache.D)
    _need(k_new, shape, cache.input_dtype, "k_new")
    _need(v_new, shape, cache.input_dtype, "v_new")
    check(lib().kv_append(ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), T, _stream(stream)),
          "kv_append")


def workspace_bytes(cache) -> int:
    return int(lib().swa_workspace_bytes(ctypes.byref(cache.desc)))


def _check_ws(ws: torch.Tensor) -> None:
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("the workspace must be a contiguous GPU tensor")


def _workspace(cache, ws: Optional[torch.Tensor]) -> torch.Tensor:
    """The cache's own workspace, or a caller's after checking it is GPU memory
    (its size is checked by the C ABI)."""
    if ws is None:
        return cache.workspace()
    _check_ws(ws)
    return ws


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check_ws(ws)
    check(lib().swa_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
          "swa_workspace_init")


def decode_attn(cache, q: torch.Tensor, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``decode_attn``: fp32 output [B, H, D] for one query per sequence."""
    _need(q, (cache.B, cache.H, cache.D), cache.input_dtype, "q")
    if out is None:
        out = torch.empty((cache.B, cache.H, cache.D), dtype=torch.float32, device=q.device)
    _need(out, (cache.B, cache.H, cache.D), torch.float32, "out")
    ws = _workspace(cache, ws)
    check(lib().decode_attn(ctypes.byref(cache.desc), _ptr(q), _ptr(out), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)), "decode_attn")
    return out


def decode_attn_int8_witness(cache, q: torch.Tensor, out: Optional[torch.Tensor] = None,
                             cmax: Optional[torch.Tensor] = None, c_all: Optional[torch.Tensor] = None,
                             want_c_all: bool = False, ws: Optional[torch.Tensor] = None,
                             stream=None):
    """``decode_attn_int8_witness``: returns (out [B,H,D], cmax [B,H], c_all [B,H,W] or None)."""
    _need(q, (cache.B, cache.H, cache.D), torch.bfloat16, "q")
    dev = q.device
    if out is None:
        out = torch.empty((cache.B, cache.H, cache.D), dtype=torch.float32, device=dev)
    if cmax is None:
        cmax = torch.empty((cache.B, cache.H), dtype=torch.float32, device=dev)
    if c_all is None and want_c_all:
        c_all = torch.empty((cache.B, cache.H, cache.W), dtype=torch.float32, device=dev)
    _need(out, (cache.B, cache.H, cache.D), torch.float32, "out")
    _need(cmax, (cache.B, cache.H), torch.float32, "cmax")
    if c_all is not None:
        _need(c_all, (cache.B, cache.H, cache.W), torch.float32, "c_all")
    ws = _workspace(cache, ws)
    check(lib().decode_attn_int8_witness(ctypes.byref(cache.desc), _ptr(q), _ptr(out), _ptr(cmax),
                                         _ptr(c_all), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)), "decode_attn_int8_witness")
    return out, cmax, c_all


def decode_attn_int8_witness_tv(cache, q: torch.Tensor, tau: float = 0.2, out: Optional[torch.Tensor] = None,
                                cmax: Optional[torch.Tensor] = None, tv: Optional[torch.Tensor] = None,
                                gate: Optional[torch.Tensor] = None, want_c_all: bool = False,
                                ws: Optional[torch.Tensor] = None, stream=None):
    """``decode_attn_int8_witness_tv``: returns (out, cmax, tv [B,H], gate [B,H] int32, c_all or None)."""
    _need(q, (cache.B, cache.H, cache.D), torch.bfloat16, "q")
    dev = q.device
    BH = (cache.B, cache.H)
    out = torch.empty((cache.B, cache.H, cache.D), dtype=torch.float32, device=dev) if out is None else out
    cmax = torch.empty(BH, dtype=torch.float32, device=dev) if cmax is None else cmax
    tv = torch.empty(BH, dtype=torch.float32, device=dev) if tv is None else tv
    gate = torch.empty(BH, dtype=torch.int32, device=dev) if gate is None else gate
    c_all = torch.empty((cache.B, cache.H, cache.W), dtype=torch.float32, device=dev) if want_c_all else None
    _need(out, (cache.B, cache.H, cache.D), torch.float32, "out")
    for t, name, dt in ((cmax, "cmax", torch.float32), (tv, "tv", torch.float32), (gate, "gate", torch.int32)):
        _need(t, BH, dt, name)
    ws = _workspace(cache, ws)
    check(lib().decode_attn_int8_witness_tv(ctypes.byref(cache.desc), _ptr(q), _ptr(out), _ptr(cmax), _ptr(tv),
                                            _ptr(gate), float(tau), _ptr(c_all), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream)),
          "decode_attn_int8_witness_tv")
    return out, cmax, tv, gate, c_all


def decode_attn_int8_dither(cache, q: torch.Tensor, delta: float, tau: float = 0.2,
                            out: Optional[torch.Tensor] = None, cert: Optional[torch.Tensor] = None,
                            tv: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
                            want_tv: bool = True, ws: Optional[torch.Tensor] = None, stream=None):
    """``decode_attn_int8_dither``: returns (out [B,H,D], cert [B,H], tv, gate) -- tv and gate
    are None when ``want_tv`` is false.  ``delta`` is the failure budget of one (sequence, head)."""
    _need(q, (cache.B, cache.H, cache.D), torch.bfloat16, "q")
    dev = q.device
    BH = (cache.B, cache.H)
    out = torch.empty((cache.B, cache.H, cache.D), dtype=torch.float32, device=dev) if out is None else out
    cert = torch.empty(BH, dtype=torch.float32, device=dev) if cert is None else cert
    if want_tv:
        tv = torch.empty(BH, dtype=torch.float32, device=dev) if tv is None else tv
        gate = torch.empty(BH, dtype=torch.int32, device=dev) if gate is None else gate
    _need(out, (cache.B, cache.H, cache.D), torch.float32, "out")
    _need(cert, BH, torch.float32, "cert")
    if tv is not None:
        _need(tv, BH, torch.float32, "tv")
    if gate is not None:
        _need(gate, BH, torch.int32, "gate")
    ws = _workspace(cache, ws)
    check(lib().decode_attn_int8_dither(ctypes.byref(cache.desc), _ptr(q), _ptr(out), _ptr(cert), _ptr(tv),
                                        _ptr(gate), float(tau), float(delta), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)),
          "decode_attn_int8_dither")
    return out, cert, tv, gate


def decode_step(cache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``decode_step``: append one token per sequence ([B, H, 1, D]) and decode ``q`` in one
    call (bf16 / fp32 kinds).  Returns out [B, H, D] fp32."""
    shape = (cache.B, cache.H, 1, cache.D)
    _need(k_new, shape, cache.input_dtype, "k_new")
    _need(v_new, shape, cache.input_dtype, "v_new")
    _need(q, (cache.B, cache.H, cache.D), cache.input_dtype, "q")
    if out is None:
        out = torch.empty((cache.B, cache.H, cache.D), dtype=torch.float32, device=q.device)
    _need(out, (cache.B, cache.H, cache.D), torch.float32, "out")
    ws = _workspace(cache, ws)
    check(lib().decode_step(ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)), "decode_step")
    return out


def decode_step_int8(cache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, tau: float = 0.2,
                     delta: float = 1e-6, want_tv: bool = False, out: Optional[torch.Tensor] = None,
                     cmax: Optional[torch.Tensor] = None, tv: Optional[torch.Tensor] = None,
                     gate: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """``decode_step_int8``: append one token per sequence ([B, H, 1, D] bf16) and decode ``q``
    in one call (INT8 kinds).  Returns (out [B,H,D], cmax [B,H], tv, gate); tv and gate are None
    unless ``want_tv`` or passed in.  ``cmax`` is the certificate for "int8_dither"."""
    shape = (cache.B, cache.H, 1, cache.D)
    _need(k_new, shape, torch.bfloat16, "k_new")
    _need(v_new, shape, torch.bfloat16, "v_new")
    _need(q, (cache.B, cache.H, cache.D), torch.bfloat16, "q")
    dev = q.device
    BH = (cache.B, cache.H)
    out = torch.empty((cache.B, cache.H, cache.D), dtype=torch.float32, device=dev) if out is None else out
    cmax = torch.empty(BH, dtype=torch.float32, device=dev) if cmax is None else cmax
    if want_tv:
        tv = torch.empty(BH, dtype=torch.float32, device=dev) if tv is None else tv
        gate = torch.empty(BH, dtype=torch.int32, device=dev) if gate is None else gate
    _need(out, (cache.B, cache.H, cache.D), torch.float32, "out")
    _need(cmax, BH, torch.float32, "cmax")
    if tv is not None:
        _need(tv, BH, torch.float32, "tv")
    if gate is not None:
        _need(gate, BH, torch.int32, "gate")
    ws = _workspace(cache, ws)
    check(lib().decode_step_int8(ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), _ptr(cmax),
                                 _ptr(tv), _ptr(gate), float(tau), float(delta), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)), "decode_step_int8")
    return out, cmax, tv, gate


def decode_step_int8_static(cache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, tau: float = 0.2,
                            delta: float = 1e-6, out: Optional[torch.Tensor] = None,
                            cmax: Optional[torch.Tensor] = None, tv: Optional[torch.Tensor] = None,
                            gate: Optional[torch.Tensor] = None, stream=None):
    """``decode_step_int8_static``: ``decode_step_int8`` with the split partials in the
    library's static device scratch (no workspace).  The caller passes every output
    tensor it wants written (``out`` and ``cmax`` are allocated here if not given, so a
    caller that must not allocate passes them).  Returns (out, cmax, tv, gate)."""
    shape = (cache.B, cache.H, 1, cache.D)
    _need(k_new, shape, torch.bfloat16, "k_new")
    _need(v_new, shape, torch.bfloat16, "v_new")
    _need(q, (cache.B, cache.H, cache.D), torch.bfloat16, "q")
    dev = q.device
    BH = (cache.B, cache.H)
    out = torch.empty((cache.B, cache.H, cache.D), dtype=torch.float32, device=dev) if out is None else out
    cmax = torch.empty(BH, dtype=torch.float32, device=dev) if cmax is None else cmax
    _need(out, (cache.B, cache.H, cache.D), torch.float32, "out")
    _need(cmax, BH, torch.float32, "cmax")
    if tv is not None:
        _need(tv, BH, torch.float32, "tv")
    if gate is not None:
        _need(gate, BH, torch.int32, "gate")
    check(lib().decode_step_int8_static(ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                        _ptr(cmax), _ptr(tv), _ptr(gate), float(tau), float(delta),
                                        _stream(stream)), "decode_step_int8_static")
    return out, cmax, tv, gate


def kv_truncate(cache, cut: torch.Tensor, stream=None) -> torch.Tensor:
    """``kv_truncate``: returns ok [B] int32 (1 truncated, 0 must recompute)."""
    _need(cut, (cache.B,), torch.int32, "cut")
    ok = torch.empty((cache.B,), dtype=torch.int32, device=cut.device)
    check(lib().kv_truncate(ctypes.byref(cache.desc), _ptr(cut), _ptr(ok), _stream(stream)), "kv_truncate")
    return ok


def validate(cache, stream=None) -> int:
    """``swa_validate``: number of slots violating the position invariant (syncs)."""
    viol = torch.zeros((1,), dtype=torch.int32, device=cache.k.device)
    check(lib().swa_validate(ctypes.byref(cache.desc), _ptr(viol), _stream(stream)), "swa_validate")
    return int(viol.item())


def status_string(status: int) -> str:
    return _capi.status_string(status)
