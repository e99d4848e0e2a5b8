"""Sliding-window ring-buffer KV cache and decode attention for AMD MI355X (gfx950).

The decode step (append k_t/v_t into a ring of W slots that records absolute
positions, then single-query attention over exactly the last W tokens; an
INT8 variant also emits the band-norm witness bound, and an INT8 variant
with subtractive dither emits a probabilistic bound) runs in hand-written HIP
kernels behind the C ABI of ``include/swa.h`` (``libswa.so``).  This package
is the thin Python binding: torch supplies device memory and the stream.
"""

from ._capi import EXPORTS, SwaError, lib
from .cache import (KVCache, SeqView, cache_reset, decode_attn, decode_attn_int8_dither, decode_step, decode_step_int8,
                    decode_step_int8_static, decode_attn_int8_witness, decode_attn_int8_witness_tv, kv_append,
                    kv_truncate, status_string, validate, workspace_bytes, workspace_init)

__all__ = ["KVCache", "SeqView", "SwaError", "EXPORTS", "lib", "cache_reset", "kv_append",
           "decode_attn", "decode_attn_int8_witness", "decode_attn_int8_witness_tv",
           "decode_attn_int8_dither", "decode_step", "decode_step_int8", "decode_step_int8_static",
           "workspace_bytes",
           "workspace_init", "kv_truncate",
           "validate", "status_string"]
