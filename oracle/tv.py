"""Total-variation bound on the attention weights from the logit-error bound.

[WitCert] "为什么在线监控 KV 误差如此困难" section: earlier runtime work bounds
the total variation (TV) of the attention distribution by tanh of the largest
logit error, independent of the data; the "SGLang 生产级落地" section has the
decode pass emit a per-step TV upper bound next to its output; the Tier A
discussion ("频带酉性与双层证书") calls a step dangerous when TV > 0.2.

Reading taken (the tight constant is not printed on the pages): if every
visible logit moves by at most E, TV <= tanh(E/2).  The bound is attained by
moving a set of probability mass 1/(1+e^E) up by E and the rest down by E,
so no smaller function of E alone is sound; tanh(E) (the pages' prior form)
is also sound and looser.  With E = max_t c_t the bound covers the
quantization of the keys (values do not move the weights).

Test infrastructure only (see the package docstring).
"""

from __future__ import annotations

import numpy as np

from . import int8 as oint8
from .attention import softmax_weights

DANGER_TV = 0.2


def tv_distance(p: np.ndarray, q: np.ndarray) -> float:
    """Half the L1 distance between two distributions."""
    return 0.5 * float(np.sum(np.abs(np.asarray(p, dtype=np.float64) - np.asarray(q, dtype=np.float64))))


def tv_bound(e: float) -> float:
    """Tight TV bound for logit perturbations of size at most e: tanh(e/2)."""
    return float(np.tanh(0.5 * float(e)))


def prior_tv_bound(e: float) -> float:
    """The data-independent form quoted as prior work: tanh(e)."""
    return float(np.tanh(float(e)))


def max_tv_over_signs(p: np.ndarray, e: float) -> float:
    """Largest TV over perturbations with every component +e or -e
    (brute force over all 2^n sign patterns; tiny n only)."""
    p = np.asarray(p, dtype=np.float64)
    n = p.size
    best = 0.0
    logp = np.log(p)
    for mask in range(1 << n):
        eps = np.array([e if (mask >> j) & 1 else -e for j in range(n)])
        best = max(best, tv_distance(p, softmax_weights(logp + eps)))
    return best


def int8_attention_tv(q: np.ndarray, k: np.ndarray, v: np.ndarray, next_position: int, w: int) -> dict:
    """True TV between the attention weights over the exact keys and over the
    INT8 cache's keys (dequantized blocks, exact staged tokens), plus the
    bound tanh(cmax/2) from the witness."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    res = oint8.int8_decode(q, k, v, next_position, w)
    pos = res["positions"]
    d = q.shape[-1]
    nb = next_position // oint8.BLOCK
    ks, kc = res["k_scales"], res["k_codes"]
    k_hat = k[pos].copy()
    for i, p in enumerate(pos):
        if p < nb * oint8.BLOCK:
            k_hat[i] = oint8.dequantize(kc[p], ks[p // oint8.BLOCK])
    if pos.size == 0:
        return {"tv": 0.0, "bound": 0.0, "cmax": 0.0}
    p_exact = softmax_weights((k[pos] @ q) / np.sqrt(d))
    p_quant = softmax_weights((k_hat @ q) / np.sqrt(d))
    return {"tv": tv_distance(p_exact, p_quant), "bound": tv_bound(res["cmax"]), "cmax": res["cmax"],
            "emax": float(np.max(res["e"]))}
