"""CPU oracle for the sliding-window ring-buffer decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing); the
only thing both sides consume is the raw input data produced by the seeded
generators in ``workloads/``, which hold none of the method's arithmetic.

Everything here is plain, slow and meant to be read against the pages:
NumPy float64 for attention and norms, NumPy float32 only where the method
itself fixes float32 steps (the INT8 block scale and code rounding), and plain
Python lists for the list model.

Pages cited (by title and section; the text of each is public):

* [Lean-SWA]  "用Lean4形式化验证滑动窗口KV Cache的正确性"
  (www.framerc.cn/news/4505248) -- the list model ``lastWindow``/``step``/
  ``run``, the position invariant, the ring-buffer interpretation
  ``ringToList`` and the masked full-history reference attention.
* [Prefix-Reuse]  "LLM 機制實驗（五）：改了歷史，能否只重算變化的後綴？"
  (huhohoo.com/zh-TW/docs/llm/longest-prefix-reuse) -- the cache record
  (K, V, per-row absolute positions, ``next_position``) and the window-4
  example.
* [KV-Loop]  "【AI 工业核题 D4】KV Cache 自回归生成推理（增量更新与状态拼接）"
  (airsota.com/?p=549) -- prefill/decode phases and the single-query decode
  step (write, slice, scaled dot product, max-subtracted softmax, weighted V).
* [WitCert]  "WitCert：运行时误差仪表盘，把崩溃的KV量化从22.8拉回79.7"
  (agifrontier.github.io/tutorials/witcert-sound-runtime-risk-observability-
  and-gating-for-kv-cache-quantization/) -- RoPE band unitarity, the band-norm
  witness ``w_{t,b}``, the logit-error bound ``c_t`` and the block-scale fold.

Readings taken where the pages are silent or garbled are listed where they are
used; every one is also listed in the repository's design notes.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against facts the pages and mathematics fix (worked examples, closed forms,
brute force, an independent library routine).  None is "parity unpinned".
"""

from . import bits, listmodel, attention, int8, rope, decoder, tv, reuse  # noqa: F401
