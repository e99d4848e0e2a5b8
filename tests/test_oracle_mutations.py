"""Planted bugs in the oracle must fail its pins.

The oracle is trusted only because the pins in ``tests/test_oracle_*.py`` and
``tests/test_negative_controls.py`` tie it to facts the pages and mathematics
fix.  This test checks that those pins have teeth: for each entry below it
copies ``oracle/`` and the pin tests into a temporary directory, plants one
plausible mistake in the copy (a dropped scale, an off-by-one in the window or
the ring, a swapped operand, a wrong rounding rule, a wrong Philox round...),
runs the pins there, and requires them to fail.  The same is done for the
comparisons the GPU parity tests use (``tests/parity_checks.py`` and the
ring check of ``tests/gpu_util.py``): with any one assertion taken out, a
negative control in ``tests/test_negative_controls.py`` must fail.  The
unmodified copy must pass, so a failure is the planted bug's doing.  The repository itself is
never modified, and nothing here touches the HIP library or a GPU.

Following [Lean-SWA] §6.4 (the specification serves as the oracle, and the
checker must be shown to reject wrong implementations) and the negative
controls of [Prefix-Reuse] (the "27 例" table keeps deliberately broken
reuse paths to prove the comparison can fail).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

from tests.conftest import ROOT

PIN_TESTS = sorted(f for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py") and f != "test_oracle_mutations.py")
PIN_TESTS.append("test_negative_controls.py")

# (file, exact text, planted replacement).  Each text occurs exactly once.
MUTATIONS = [
    # masked attention and its window
    ("oracle/attention.py", "scores = (k @ q) / np.sqrt(d)\n    return softmax_weights(scores) @ v",
     "scores = (k @ q)\n    return softmax_weights(scores) @ v"),
    ("oracle/attention.py", "return (pos >= t - w + 1) & (pos <= t)", "return (pos > t - w + 1) & (pos <= t)"),
    ("oracle/attention.py", "return (pos >= t - w + 1) & (pos <= t)", "return (pos >= t - w) & (pos <= t)"),
    ("oracle/attention.py", "scores = np.where(vis, (k @ q) / np.sqrt(d), -np.inf)",
     "scores = np.where(vis, (k @ q) / d, -np.inf)"),
    ("oracle/attention.py",
     "scores = np.where(vis, (k @ q) / np.sqrt(d), -np.inf)\n    return softmax_weights(scores) @ v",
     "scores = np.where(vis, (k @ q) / np.sqrt(d), -np.inf)\n    return softmax_weights(scores) @ k"),
    # INT8 quantizer, witness and INT8 decode
    ("oracle/int8.py", "return np.float32(a / np.float32(QMAX))", "return np.float32(a / np.float32(128))"),
    ("oracle/int8.py", "q = np.rint(x32 / np.float32(s))", "q = np.floor(x32 / np.float32(s) + np.float32(0.5))"),
    ("oracle/int8.py", "q = np.rint(x32 / np.float32(s))", "q = np.rint(x32 * (np.float32(1) / np.float32(s)))"),
    ("oracle/int8.py", "xb = x.reshape(x.shape[:-1] + (d // band, band))",
     "xb = np.swapaxes(x.reshape(x.shape[:-1] + (band, d // band)), -1, -2)"),
    ("oracle/int8.py", "return (np.asarray(w, dtype=np.float64) @ nq) / np.sqrt(q.shape[-1])",
     "return (np.asarray(w, dtype=np.float64) @ nq)"),
    ("oracle/int8.py", "return np.abs(r @ q) / np.sqrt(q.shape[-1])", "return np.abs(r @ q)"),
    ("oracle/int8.py", "nb = n // BLOCK\n    nq",
     "nb = (n + BLOCK - 1) // BLOCK if n % BLOCK > 8 else n // BLOCK\n    nq"),
    ("oracle/int8.py", "ln = min(w, n)\n    vis", "ln = min(w - 1, n)\n    vis"),
    ("oracle/int8.py", "r = k[:n] - k_hat", "r = k_hat - k[:n] * 0.999"),
    # list model and ring interpretation
    ("oracle/listmodel.py", "if w < len(c2):", "if w <= len(c2):"),
    ("oracle/listmodel.py", "return list(hs[n - min(w, n):])", "return list(hs[max(n - w - 1, 0):])"),
    ("oracle/listmodel.py", "start = next_position - ln\n    return [buf[(start + i) % w]",
     "start = next_position - w\n    return [buf[(start + i) % w]"),
    ("oracle/listmodel.py", "return [p - ln + 1 + i for i in range(ln)]", "return [p - w + 1 + i for i in range(ln)]"),
    ("oracle/listmodel.py", "rhs = list(xs)[max(n + 1 - w, 0):] + [kv]", "rhs = list(xs)[max(n - w, 0):] + [kv]"),
    ("oracle/listmodel.py", "return pos % w", "return (pos + 1) % w"),
    # full-history decoder and the expected INT8 ring store
    ("oracle/decoder.py", "t = self._n - 1\n        return", "t = self._n\n        return"),
    ("oracle/decoder.py", "k_scale[s // blk] = ks[j // blk]", "k_scale[s // blk] = ks[s // blk]"),
    ("oracle/decoder.py", "staged = list(range(nb * blk, n))", "staged = list(range(nb * blk, n + 1))"),
    ("oracle/decoder.py", "v_codes[s] = vc[j]", "v_codes[s] = kc[j]"),
    ("oracle/decoder.py", "v_scale[s // blk] = vs[j // blk]", "v_scale[s // blk] = ks[j // blk]"),
    ("oracle/decoder.py", "k_codes[s] = kc[j]", "k_codes[s] = kc[s]"),
    ("oracle/decoder.py", "r = np.asarray(k[j], dtype=np.float64) - int8.dequantize(kc[j], ks[j // blk])",
     "r = np.asarray(k[j], dtype=np.float64) - int8.dequantize(kc[j], vs[j // blk])"),
    ("oracle/decoder.py", "r = np.asarray(k[j], dtype=np.float64) - int8.dequantize(kc[j], ks[j // blk])",
     "r = np.asarray(k[j], dtype=np.float32) - int8.dequantize(kc[j], ks[j // blk]).astype(np.float32)"),
    # RoPE and bf16 bits
    ("oracle/rope.py", "out[..., 1::2] = a * s + b * c", "out[..., 1::2] = a * s - b * c"),
    ("oracle/rope.py", "theta = base ** (-2.0 * i / d)", "theta = base ** (-1.0 * i / d)"),
    ("oracle/bits.py", "<< np.uint32(16)", "<< np.uint32(15)"),
    # TV bound
    ("oracle/tv.py", "return float(np.tanh(0.5 * float(e)))", "return float(np.tanh(float(e)))"),
    ("oracle/tv.py", "return float(np.tanh(0.5 * float(e)))", "return float(np.tanh(0.25 * float(e)))"),
    ("oracle/tv.py", "return 0.5 * float(np.sum(np.abs(", "return float(np.sum(np.abs("),
    ("oracle/tv.py", "k_hat[i] = oint8.dequantize(kc[p], ks[p // oint8.BLOCK])", "k_hat[i] = k[p]"),
    ("oracle/tv.py", "p_quant = softmax_weights((k_hat @ q) / np.sqrt(d))", "p_quant = softmax_weights((k_hat @ q) / d)"),
    # prefix-reuse truncation
    ("oracle/reuse.py", "return max(0, min(n, len(new) - 1))", "return max(0, min(n, len(new)))"),
    ("oracle/reuse.py", "if n > w and cut not in (0, n):", "if n > w and cut != n:"),
    ("oracle/reuse.py", "if n > w and cut not in (0, n):", "if n >= w and cut not in (0, n):"),
    ("oracle/reuse.py", "if int8 and cut % 16 != 0 and cut < 16 * (n // 16):", "if int8 and cut % 16 != 0:"),
    ("oracle/reuse.py", "if cut < 0 or cut > n:", "if cut < 0:"),
    # Philox-4x32-10 and the Tier B dither
    ("oracle/philox.py",
     "x0, x1, x2, x3 = ((p1 >> width) ^ x1 ^ k0, p1 & mask, (p0 >> width) ^ x3 ^ k1, p0 & mask)",
     "x0, x1, x2, x3 = ((p1 >> width) ^ x3 ^ k0, p1 & mask, (p0 >> width) ^ x1 ^ k1, p0 & mask)"),
    ("oracle/philox.py", "k0 = (k0 + c0) & mask", "k0 = (k0 + c1) & mask"),
    ("oracle/philox.py",
     "x0, x1, x2, x3 = ((p1 >> sh) ^ x1 ^ k0, p1 & lo32, (p0 >> sh) ^ x3 ^ k1, p0 & lo32)",
     "x0, x1, x2, x3 = ((p1 >> sh) ^ x1 ^ k0, p0 & lo32, (p0 >> sh) ^ x3 ^ k1, p1 & lo32)"),
    ("oracle/philox.py", "k1 = (k1 + c1) & lo32", "k1 = (k1 + c0) & lo32"),
    ("oracle/dither.py", "return np.array([position, group, head, layer], dtype=np.uint64)",
     "return np.array([position, group, layer, head], dtype=np.uint64)"),
    ("oracle/dither.py", "ctr[i, g] = philox_counter(layer, head, int(p), g)",
     "ctr[i, g] = philox_counter(head, layer, int(p), g)"),
    ("oracle/dither.py", "ctr[i, g] = philox_counter(layer, head, int(p), g)",
     "ctr[i, g] = philox_counter(layer, head, int(p) + 1, g)"),
    ("oracle/dither.py", '.astype("<u4").view(np.uint8)', '.astype(">u4").view(np.uint8)'),
    ("oracle/dither.py", "return np.array([r & 0xFFFFFFFF, r >> 32]", "return np.array([r >> 32, r & 0xFFFFFFFF]"),
    ("oracle/dither.py", "return 0.5 - (np.asarray(m, dtype=np.float64) + 0.5) / LEVELS",
     "return 0.5 - np.asarray(m, dtype=np.float64) / LEVELS"),
    ("oracle/dither.py", "return 0.5 - (np.asarray(m, dtype=np.float64) + 0.5) / LEVELS",
     "return (np.asarray(m, dtype=np.float64) + 0.5) / LEVELS - 0.5"),
    ("oracle/dither.py", "return np.clip(np.rint(t), -QMAX, QMAX)",
     "return np.clip(np.floor(t + np.float32(0.5)), -QMAX, QMAX)"),
    ("oracle/dither.py", "t = y + np.asarray(u, dtype=np.float32)", "t = y - np.asarray(u, dtype=np.float32)"),
    ("oracle/dither.py", "(np.asarray(codes, dtype=np.float64) - np.asarray(u, dtype=np.float64))",
     "(np.asarray(codes, dtype=np.float64) + np.asarray(u, dtype=np.float64))"),
    ("oracle/dither.py", "np.sqrt(np.log(2.0 * n_q / delta) / 6.0)", "np.sqrt(np.log(2.0 * n_q / delta) / 2.0)"),
    ("oracle/dither.py", "np.sqrt(np.log(2.0 * n_q / delta) / 6.0)", "np.sqrt(np.log(n_q / delta) / 6.0)"),
    ("oracle/dither.py", "return s_tok / np.sqrt(d) * f", "return s_tok / d * f"),
    ("oracle/dither.py", "BETA = 2.0 ** -9 + 2.0 ** -16", "BETA = 2.0 ** -16"),
    ("oracle/dither.py", "n_q = int(np.count_nonzero(quantized))", "n_q = ln"),
    ("oracle/dither.py", "vs, vc = quantize_history(v[:nq_all], nb, u)",
     "vs, vc = quantize_history(v[:nq_all], nb, dither_values(dither_bytes(request, layer, head + 1, "
     "np.arange(nq_all), d)))"),
    ("oracle/dither.py", "k_hat[rows] = dequantize(kc[rows], ks[blk], u[rows])",
     "k_hat[rows] = dequantize(kc[rows], ks[blk], 0 * u[rows])"),
    ("oracle/dither.py", "v_hat[rows] = dequantize(vc[rows], vs[blk], u[rows])",
     "v_hat[rows] = dequantize(vc[rows], vs[blk], 0 * u[rows])"),
    ("oracle/dither.py", "e = np.abs((k[vis] - k_hat[vis]) @ q) / np.sqrt(d)",
     "e = np.abs((k[vis] - k_hat[vis]) @ q) / d"),
    ("oracle/dither.py", "quantized = vis < nq_all", "quantized = vis <= nq_all"),
    ("oracle/int8.py", "        return np.zeros(x32.shape, dtype=np.int8)", "        return np.ones(x32.shape, dtype=np.int8)"),
    ("oracle/int8.py", "out = softmax_weights((k_hat[vis] @ q) / np.sqrt(d)) @ v_hat[vis]",
     "out = softmax_weights((k_hat[vis] @ q) / np.sqrt(d)) @ v[vis]"),
    ("oracle/int8.py", "out = softmax_weights((k_hat[vis] @ q) / np.sqrt(d)) @ v_hat[vis]",
     "out = softmax_weights((k[vis] @ q) / np.sqrt(d)) @ v_hat[vis]"),
    ("oracle/int8.py", '"cmax": float(np.max(c)) if ln else 0.0', '"cmax": float(np.max(e)) if ln else 0.0'),
    ("oracle/int8.py", "vis = np.arange(t - ln + 1, t + 1, dtype=np.int64)", "vis = np.arange(t - ln, t, dtype=np.int64)"),
    ("oracle/int8.py", "return np.sqrt(np.sum(xb * xb, axis=-1))", "return np.sum(np.abs(xb), axis=-1)"),
    ("oracle/attention.py", "    if k.shape[0] == 0:\n        return np.zeros(v.shape[-1], dtype=np.float64)",
     "    if k.shape[0] == 0:\n        return np.ones(v.shape[-1], dtype=np.float64)"),
    ("oracle/attention.py", "    if not np.any(vis):\n        return np.zeros(v.shape[-1], dtype=np.float64)",
     "    if not np.any(vis):\n        return np.ones(v.shape[-1], dtype=np.float64)"),
    ("oracle/attention.py", "return (pos >= t - w + 1) & (pos <= t)", "return (pos >= t - w + 1) & (pos < t)"),
    ("oracle/decoder.py", "attention.masked_attention(q[h], pos, k[h], v[h], t, w)",
     "attention.masked_attention(q[h], pos, k[h], v[h], t, w + 1)"),
    ("oracle/decoder.py", "idx = listmodel.last_window(w, list(range(self._n)))",
     "idx = listmodel.last_window(w - 1, list(range(self._n)))"),
    ("oracle/decoder.py", "wit[s] = int8.band_norms(r, band)", "wit[s] = int8.band_norms(r, band) * 1.001"),
    ("oracle/tv.py", "if p < nb * oint8.BLOCK:", "if p < (nb - 1) * oint8.BLOCK:"),
    ("oracle/tv.py", "p_exact = softmax_weights((k[pos] @ q) / np.sqrt(d))", "p_exact = softmax_weights((k[pos] @ q) / d)"),
    ("oracle/rope.py", "out[..., 0::2] = a * c - b * s", "out[..., 0::2] = a * c + b * s"),
    ("oracle/reuse.py", "        if a != b:\n            break", "        if a != b:\n            continue"),
    ("oracle/listmodel.py", "    if w < len(c2):\n        return c2[1:]", "    if w < len(c2):\n        return c2[:-1]"),
    ("oracle/listmodel.py", "    return all(pos_of(cell) == base + i for i, cell in enumerate(c))",
     "    return all(pos_of(cell) >= base for i, cell in enumerate(c))"),
    ("oracle/philox.py", "    for _ in range(rounds):\n        p0 = m0 * x0\n        p1 = m1 * x2\n        x0, x1, x2, x3 = ((p1 >> width)",
     "    for _ in range(rounds - 1):\n        p0 = m0 * x0\n        p1 = m1 * x2\n        x0, x1, x2, x3 = ((p1 >> width)"),
    ("oracle/philox.py", "    for _ in range(rounds):\n        p0 = m0 * x0\n        p1 = m1 * x2\n        x0, x1, x2, x3 = ((p1 >> sh)",
     "    for _ in range(rounds - 1):\n        p0 = m0 * x0\n        p1 = m1 * x2\n        x0, x1, x2, x3 = ((p1 >> sh)"),
    ('oracle/dither.py',
     'out = softmax_weights((k_hat[vis] @ q) / np.sqrt(d)) @ v_hat[vis]\n    return {\n        "out": out,\n        "positions": vis,\n        "e": e,',
     'out = softmax_weights((k_hat[vis] @ q) / np.sqrt(d)) @ v[vis]\n    return {\n        "out": out,\n        "positions": vis,\n        "e": e,'),
    ('oracle/dither.py',
     '+ np.sum(np.abs(q)) * BETA',
     '+ np.linalg.norm(q) * BETA'),
    ('oracle/listmodel.py',
     '    if p < 0:\n        return []',
     '    if p < 0:\n        return [0]'),
    ('oracle/reuse.py',
     '    return max(0, min(n, len(new) - 1))',
     '    return min(n, len(new) - 1)'),
    ('oracle/bits.py',
     '    if x.dtype == np.uint16:\n        return bf16_to_f64(x)',
     '    if x.dtype == np.uint16:\n        return x.astype(np.float64)'),
    ('oracle/tv.py',
     '    if pos.size == 0:\n        return {"tv": 0.0, "bound": 0.0, "cmax": 0.0}',
     '    if pos.size == 0:\n        return {"tv": 0.0, "bound": 1.0, "cmax": 0.0}'),
    ('oracle/dither.py',
     '        "cert": float(np.max(c)) if ln else 0.0,',
     '        "cert": float(np.max(e)) if ln else 0.0,'),
    ('oracle/dither.py',
     '        s_tok[rows] = np.float64(ks[blk])',
     '        s_tok[rows] = np.float64(vs[blk])'),
    ('oracle/dither.py',
     'f = np.linalg.norm(q) * np.sqrt',
     'f = np.sum(np.abs(q)) * np.sqrt'),
    ('oracle/dither.py',
     '    for g in range(groups):\n        for i, p in enumerate(pos):\n            ctr[i, g] = philox_counter(layer, head, int(p), g)',
     '    for g in range(groups):\n        for i, p in enumerate(pos):\n            ctr[i, g] = philox_counter(layer, head, int(p), 0)'),
    ('oracle/decoder.py',
     '        v_codes[s] = vc[j]\n',
     '        v_codes[s] = vc[j] if j % 16 else kc[j]\n'),
    ('oracle/tv.py',
     '    logp = np.log(p)\n',
     '    logp = np.log(p) * 0.5\n'),
    ('oracle/rope.py',
     '    return np.asarray(pos, dtype=np.float64)[..., None] * theta',
     '    return (np.asarray(pos, dtype=np.float64)[..., None] + 1) * theta'),
    ('oracle/attention.py',
     '    return e / np.sum(e, axis=-1, keepdims=True)',
     '    return e / (np.sum(e, axis=-1, keepdims=True) + 1e-9)'),
    ('oracle/listmodel.py',
     '    return list(c) == last_window(w, hs)',
     '    return len(c) == len(last_window(w, hs))'),
    ('oracle/listmodel.py',
     '        c = step(w, c, kv)\n    return c',
     '        c = step(w, c, kv)\n    return c[::-1] if len(c) > 3 else c'),
    ('oracle/listmodel.py',
     '    return [buf[(start + i) % w] for i in range(ln)]',
     '    return [buf[(start + i + 1) % w] for i in range(ln)]'),
    ('oracle/reuse.py',
     '    if int8 and cut % 16 != 0 and cut < 16 * (n // 16):',
     '    if int8 and cut % 8 != 0 and cut < 16 * (n // 16):'),
    ('oracle/decoder.py',
     '    idx = listmodel.ring_state(w, list(int(p) for p in positions), lambda p: p, -1)',
     '    idx = listmodel.ring_state(w, list(int(p) for p in positions)[:-1], lambda p: p, -1)'),
    ('oracle/decoder.py',
     '    nb = n // blk\n    ks, kc = int8.quantize_history(np.asarray(k)[: nb * blk], nb)',
     '    nb = (n + 1) // blk\n    ks, kc = int8.quantize_history(np.asarray(k)[: nb * blk], nb)'),
    ('oracle/int8.py',
     '    for blk in range(nb):\n        rows = slice(blk * BLOCK, (blk + 1) * BLOCK)\n        s, c = quantize_block(x[rows])',
     '    for blk in range(nb):\n        rows = slice(blk * BLOCK, (blk + 1) * BLOCK)\n        s, c = quantize_block(x[rows][::-1])'),
    ('oracle/int8.py',
     '    return np.clip(q, -QMAX, QMAX).astype(np.int8)',
     '    return np.clip(q, -QMAX + 1, QMAX).astype(np.int8)'),
    ('oracle/int8.py',
     '    return np.float64(np.float32(s)) * np.asarray(codes, dtype=np.float64)',
     '    return np.float64(np.float32(s) * np.float32(1.0000001)) * np.asarray(codes, dtype=np.float64)'),
    ('oracle/dither.py',
     '    return np.asarray(words, dtype=np.uint32).astype("<u4").view(np.uint8).reshape(-1, GROUP)',
     '    return np.asarray(words, dtype=np.uint32)[..., ::-1].astype("<u4").view(np.uint8).reshape(-1, GROUP)'),
    ('oracle/dither.py',
     '    return np.clip(np.rint(t), -QMAX, QMAX).astype(np.int8)',
     '    return np.clip(np.rint(t), -QMAX, QMAX - 1).astype(np.int8)'),
    ('oracle/dither.py',
     '    nq_all = nb * BLOCK\n',
     '    nq_all = nb * BLOCK if nb < 3 else (nb - 1) * BLOCK\n'),
    ('oracle/tv.py',
     '    for mask in range(1 << n):',
     '    for mask in range(1 << (n - 1)):'),
    ('oracle/philox.py',
     '    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85),',
     '    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE84),'),
    ('oracle/attention.py',
     '    m = np.max(scores, axis=-1, keepdims=True)',
     '    m = np.max(scores, axis=-1, keepdims=True) * 0 + np.min(np.where(np.isfinite(scores), scores, np.inf), axis=-1, keepdims=True)'),
    ('oracle/rope.py',
     '    a, b = x[..., 0::2], x[..., 1::2]\n    out = np.empty_like(x)',
     '    b, a = x[..., 0::2], x[..., 1::2]\n    out = np.empty_like(x)'),
    ('oracle/listmodel.py',
     '    lhs = (list(xs) + [kv])[max(n + 1 - w, 0):]\n    rhs = list(xs)[max(n + 1 - w, 0):] + [kv]',
     '    lhs = (list(xs) + [kv])[max(n + 1 - w, 0):]\n    rhs = list(xs)[max(n + 2 - w, 0):] + [kv]'),
    ('oracle/listmodel.py',
     '    lhs = (list(xs) + [kv])[max(n + 1 - w, 0):]\n    rhs = list(xs)[max(n - w, 0):] + [kv]',
     '    lhs = (list(xs) + [kv])[max(n + 1 - w, 0):]\n    rhs = list(xs)[max(n + 1 - w, 0):] + [kv]'),
    ('oracle/decoder.py',
     '            self._cache = (np.arange(self._n, dtype=np.int64), k, v)',
     '            self._cache = (np.arange(1, self._n + 1, dtype=np.int64), k, v)'),
    ('oracle/decoder.py',
     '        return np.stack([attention.masked_attention(q[h], pos, k[h], v[h], t, w)',
     '        return np.stack([attention.masked_attention(q[0], pos, k[h], v[h], t, w)'),
    ('oracle/attention.py',
     '    scores = np.where(vis, (k @ q) / np.sqrt(d), -np.inf)',
     '    scores = np.where(vis, (k @ q) / np.sqrt(d), -1e3)'),
    ('oracle/int8.py',
     '    xb = x.reshape(x.shape[:-1] + (d // band, band))\n    return',
     '    xb = x.reshape(x.shape[:-1] + (d // band, band))[..., ::-1, :]\n    return'),
    ('oracle/int8.py',
     '    nq = band_norms(q, band)\n',
     '    nq = band_norms(q, band)[::-1]\n'),
    ('oracle/int8.py',
     '    r = k[:n] - k_hat  # exact residual',
     '    r = k[:n] - k_hat * 1.0  # exact residual\n    r[-1] = 0'),
    ('oracle/philox.py',
     '    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),',
     '    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73A),'),
    ('oracle/dither.py',
     '    return group_bytes(words.reshape(-1, 4)).reshape(pos.size, d)',
     '    return group_bytes(words.reshape(-1, 4)[::-1]).reshape(pos.size, d)'),
    ('oracle/dither.py',
     '    assert 0 <= r < 1 << 64\n    return np.array([r & 0xFFFFFFFF, r >> 32], dtype=np.uint64)',
     '    assert 0 <= r < 1 << 64\n    return np.array([r & 0xFFFFFFFF, (r >> 32) ^ 1], dtype=np.uint64)'),
    ('oracle/dither.py',
     '        k_hat[rows] = dequantize(kc[rows], ks[blk], u[rows])',
     '        k_hat[rows] = dequantize(kc[rows], ks[blk], u[rows][::-1])'),
    ('oracle/tv.py',
     '    p_quant = softmax_weights((k_hat @ q) / np.sqrt(d))',
     '    p_quant = softmax_weights((k_hat @ q) / np.sqrt(d) * 1.0001)'),
    ('oracle/reuse.py',
     '    if n > w and cut not in (0, n):\n        return False',
     '    if n > w + 1 and cut not in (0, n):\n        return False'),
    ('oracle/rope.py',
     '    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)',
     '    return np.concatenate([a * c - b * s, a * s - b * c], axis=-1)'),
    ('oracle/dither.py',
     '    assert position0 % BLOCK == 0 and position0 >= 0\n',
     '    assert position0 % BLOCK == 0 and position0 >= 0\n    position0 = 0\n'),
    ('oracle/dither.py',
     '    c = np.where(quantized, token_bound(q, s_tok[vis], n_q, delta), 0.0)',
     '    c = np.where(quantized, token_bound(q, s_tok[vis], n_q + 1, delta), 0.0)'),
    ('oracle/dither.py',
     '    c = np.where(quantized, token_bound(q, s_tok[vis], n_q, delta), 0.0)',
     '    c = np.where(quantized, token_bound(q, s_tok[vis], n_q, delta * 2), 0.0)'),
    ('oracle/dither.py',
     '    c = np.where(quantized, token_bound(q, s_tok[vis], n_q, delta), 0.0)',
     '    c = np.where(quantized, token_bound(q, np.full(ln, s_tok[vis].max() if ln else 0.0), n_q, delta), 0.0)'),
    ('oracle/dither.py',
     '    e = np.abs((k[vis] - k_hat[vis]) @ q) / np.sqrt(d)',
     '    e = np.abs((k[vis] - k_hat[vis]) @ np.abs(q)) / np.sqrt(d)'),
    ('oracle/dither.py',
     '    return np.float64(np.float32(s)) * (np.asarray(codes, dtype=np.float64) - np.asarray(u, dtype=np.float64))',
     '    return np.float64(np.float32(s)) * (np.asarray(codes, dtype=np.float64) - np.asarray(u, dtype=np.float32).astype(np.float64) * (1 + 2.0 ** -20))'),
    ('oracle/dither.py',
     '    groups = d // GROUP\n',
     '    groups = d // GROUP\n    pos = pos + (pos >= 1000)\n'),
    ('oracle/int8.py',
     '    if ln == 0:\n        out = np.zeros(v.shape[-1], dtype=np.float64)',
     '    if ln == 0:\n        out = np.ones(v.shape[-1], dtype=np.float64)'),
    ('oracle/dither.py',
     '    if ln == 0:\n        out = np.zeros(v.shape[-1], dtype=np.float64)',
     '    if ln == 0:\n        out = np.ones(v.shape[-1], dtype=np.float64)'),
    ('oracle/dither.py',
     '        "n_q": n_q,',
     '        "n_q": ln,'),
    # The comparisons the GPU parity tests use (tests/parity_checks.py, tests/gpu_util.py): each assertion
    # taken out must let a planted difference through a negative control.
    ('tests/parity_checks.py',
     '    assert np.all(wg >= we), f"{what}: stored witness below the exact band norm"',
     '    pass'),
    ('tests/parity_checks.py',
     '    assert np.all(wg <= we * (1 + 2.0 ** -9) + 2.0 ** -24), f"{what}: stored witness not tight"',
     '    pass'),
    ('tests/parity_checks.py',
     '    np.testing.assert_array_equal(vc[live], st["v_codes"][live], err_msg=f"{what} value codes")',
     '    pass'),
    ('tests/parity_checks.py',
     '    np.testing.assert_array_equal(vs[lb], st["v_scale"][lb], err_msg=f"{what} value scales")',
     '    pass'),
    ('tests/parity_checks.py',
     '        np.testing.assert_array_equal(bits.to_f64(vsg[p % 16]), v64[p])\n\n\ndef fp16',
     '        pass\n\n\ndef fp16'),
    ('tests/parity_checks.py',
     '    assert cmax <= (res["cmax"] + slack) * (1 + 2.0 ** -9), (cmax, res["cmax"])',
     '    pass'),
    ('tests/parity_checks.py',
     '        assert np.all(cg >= e), "per-token bound below the true logit error"',
     '        pass'),
    ('tests/parity_checks.py',
     '        assert np.all(cg <= (c + slack) * (1 + 2.0 ** -9)), "per-token bound not tight"',
     '        pass'),
    ('tests/parity_checks.py',
     '        assert not np.any(np.asarray(c_all)[~vis]), "slots without a visible quantized token must be 0"',
     '        pass'),
    ('tests/parity_checks.py',
     '    assert cert <= ref * (1 + 2.0 ** -10) + 1e-30, (what, b, h, cert, ref)',
     '    pass'),
    ('tests/parity_checks.py',
     '        assert t <= tv <= min(t * (1 + 2.0 ** -18) + 1e-30, 1.0), (tv, t)',
     '        pass'),
    ('tests/parity_checks.py',
     '            assert int(gate) == int(tv > tau)',
     '            pass'),
    ('tests/gpu_util.py',
     '        np.testing.assert_array_equal(pos[b], exp)',
     '        pass'),
    ('tests/gpu_util.py',
     '        np.testing.assert_array_equal(vv[b][:, live], v_in[b][:, exp[live]])',
     '        pass'),
    ('tests/gpu_util.py',
     '        assert npos[b] == n[b], (b, npos[b], n[b])',
     '        pass'),
    ('tests/gpu_util.py',
     '        np.testing.assert_array_equal(kc[slot0:slot0 + 16], ck, err_msg=f"key codes b={b} h={h} block {kb}")',
     '        pass'),
    ('tests/gpu_util.py',
     '        np.testing.assert_array_equal(vc[slot0:slot0 + 16], cv, err_msg=f"value codes b={b} h={h} block {kb}")',
     '        pass'),
    ('tests/gpu_util.py',
     '        assert ks[slot0 // 16] == sk and vs[slot0 // 16] == sv, (kb, ks[slot0 // 16], sk)',
     '        assert ks[slot0 // 16] == sk, (kb, ks[slot0 // 16], sk)'),
    ('tests/gpu_util.py',
     '        assert ks[slot0 // 16] == sk and vs[slot0 // 16] == sv, (kb, ks[slot0 // 16], sk)',
     '        assert vs[slot0 // 16] == sv, (kb, ks[slot0 // 16], sk)'),
    ('tests/gpu_util.py',
     '    np.testing.assert_array_equal(pos, exp_pos)\n    ksg',
     '    pass\n    ksg'),
    ('tests/gpu_util.py',
     '        np.testing.assert_array_equal(bits.to_f64(ksg[p % 16]), k64[p])\n        np.testing.assert_array_equal(bits.to_f64(vsg[p % 16]), v64[p])',
     '        np.testing.assert_array_equal(bits.to_f64(vsg[p % 16]), v64[p])'),
    ('tests/gpu_util.py',
     '        np.testing.assert_array_equal(bits.to_f64(ksg[p % 16]), k64[p])\n        np.testing.assert_array_equal(bits.to_f64(vsg[p % 16]), v64[p])',
     '        np.testing.assert_array_equal(bits.to_f64(ksg[p % 16]), k64[p])'),
]


def _copy_tree(dst: str) -> None:
    ign = shutil.ignore_patterns("__pycache__", "*.pyc")
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"), ignore=ign)
    shutil.copytree(os.path.join(ROOT, "workloads"), os.path.join(dst, "workloads"), ignore=ign)
    os.makedirs(os.path.join(dst, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"), ignore=ign)
    for f in ["conftest.py", "gpu_util.py", "parity_checks.py", *PIN_TESTS]:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))


# The pin file of each module runs first, so a caught bug stops early.
_FIRST = {"attention": ["test_oracle_attention.py"], "int8": ["test_oracle_int8.py"],
          "decoder": ["test_oracle_int8.py", "test_oracle_attention.py"], "rope": ["test_oracle_int8.py"],
          "listmodel": ["test_oracle_listmodel.py"], "bits": ["test_oracle_bits.py"], "tv": ["test_oracle_tv.py"],
          "reuse": ["test_oracle_reuse.py"], "philox": ["test_oracle_dither.py"], "dither": ["test_oracle_dither.py"],
          "parity_checks": ["test_negative_controls.py"], "gpu_util": ["test_negative_controls.py"]}


def _order(mutation) -> list:
    if mutation is None:
        return PIN_TESTS
    first = _FIRST.get(os.path.splitext(os.path.basename(mutation[0]))[0], [])
    return first + [t for t in PIN_TESTS if t not in first]


def _run_pins(mutation) -> tuple:
    """Run the pin tests on a copy with ``mutation`` (or none) planted;
    returns (mutation, pytest exit code, tail of its output)."""
    with tempfile.TemporaryDirectory(prefix="oracle_mut_") as tmp:
        _copy_tree(tmp)
        if mutation is not None:
            f, text, planted = mutation
            path = os.path.join(tmp, f)
            src = open(path).read()
            assert src.count(text) == 1, (f, text)
            open(path, "w").write(src.replace(text, planted))
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                            *[os.path.join("tests", t) for t in _order(mutation)]],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
        return mutation, r.returncode, (r.stdout + r.stderr)[-600:]


def test_every_planted_bug_fails_a_pin():
    for f, text, _ in MUTATIONS:
        assert open(os.path.join(ROOT, f)).read().count(text) == 1, (f, text)
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(_run_pins, [None] + MUTATIONS))
    _, rc0, out0 = results[0]
    assert rc0 == 0, f"the unmodified oracle copy must pass its pins:\n{out0}"
    missed = [m for m, rc, _ in results[1:] if rc == 0]
    broken = [(m, rc, out) for m, rc, out in results[1:] if rc not in (0, 1)]
    assert not broken, f"pytest did not run normally on some copies: {broken[:2]}"
    assert not missed, "planted bugs no pin catches:\n" + "\n".join(f"{f}: {p!r}" for f, _, p in missed)
