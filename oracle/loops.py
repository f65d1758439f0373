"""Scalar pure-Python evaluation of the GLM-5.2 MoE layer, for tiny inputs.

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle.moe``).  A second,
independently written evaluation with explicit loops over tokens, experts and
features, using ``math.exp`` and Python floats (IEEE double).  It exists only to
cross-check ``oracle.moe`` on small cases; it shares no code with it.
Layer statement: frontier-model-atlas "GLM-5.2 model anatomy", Feed-forward /
Mixture of Experts panel.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple


def _dot(a: Sequence[float], b: Sequence[float]) -> float:
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def _mlp(xt: Sequence[float], w1, w3, w2) -> List[float]:
    F = len(w1)
    h = []
    for f in range(F):
        g = _dot(xt, w1[f])
        u = _dot(xt, w3[f])
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [_dot(w2[d], h) for d in range(len(w2))]


def layer_token(xt: Sequence[float], router_w, bias, w1, w3, w2, sw1, sw3, sw2,
                k: int, scale: float) -> Tuple[List[int], List[float], List[float]]:
    """One token: returns (selected experts in slot order, their weights, output row).

    All arguments are nested Python lists of floats (w1[e][f][d], w2[e][d][f]).
    """
    E = len(router_w)
    sig = [1.0 / (1.0 + math.exp(-_dot(xt, router_w[e]))) for e in range(E)]
    beta = [sig[e] + bias[e] for e in range(E)]
    chosen: List[int] = []
    for _ in range(k):
        best = -1
        for e in range(E):
            if e in chosen:
                continue
            if best < 0 or beta[e] > beta[best]:
                best = e
        chosen.append(best)
    total = 0.0
    for e in chosen:
        total += sig[e]
    wts = [scale * sig[e] / total for e in chosen]
    out = _mlp(xt, sw1, sw3, sw2)
    for e, wt in zip(chosen, wts):
        y = _mlp(xt, w1[e], w3[e], w2[e])
        for d in range(len(out)):
            out[d] += wt * y[d]
    return chosen, wts, out
