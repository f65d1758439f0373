"""Comparison of another implementation's results with the oracle.

TEST INFRASTRUCTURE ONLY (same import rule as ``oracle.moe``).  Takes plain
NumPy arrays; knows nothing of how they were produced.

Routing rule: expert indices must equal the oracle's, slot for slot, except on
tokens where the oracle's biased scores leave the choice open within
``tie_eps`` (the k-th / (k+1)-th gap for the set, adjacent gaps for the slot
order).  Such tokens are counted, the other implementation's choice is checked
to be a valid top-k under the oracle's scores up to ``tie_eps``, and the layer
output for them is compared against the oracle evaluated on that choice.
Tests that build exact ties on purpose (bit-identical scores) assert
``exact == tokens`` themselves: an exact tie must go to the lower index on both
sides, so it is never left to this rule.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from . import moe, mx


@dataclasses.dataclass
class RoutingReport:
    tokens: int
    exact: int
    excused: int                 # near-tie tokens whose choice differs but is valid
    invalid: List[int]           # tokens whose choice is wrong
    forced_idx: np.ndarray       # oracle idx, with excused tokens replaced by the tested choice
    max_weight_err: float        # vs the oracle's weights on forced_idx
    weight_sum_err: float        # max |sum_j w - scale|

    @property
    def ok(self) -> bool:
        return not self.invalid


def _near_topk(b: np.ndarray, sel: np.ndarray, k: int, tie_eps: float) -> bool:
    """``sel`` (slot order) is a top-k of the scores ``b`` up to ``tie_eps``."""
    chosen = b[sel]
    kth = -np.sort(-b)[k - 1]
    rest = np.delete(b, sel)
    return bool(chosen.min() >= kth - tie_eps
                and (rest.size == 0 or rest.max() <= chosen.min() + tie_eps)
                and (np.diff(chosen) <= tie_eps).all())


def _valid_choice(b: np.ndarray, sel: np.ndarray, k: int, n_group: int, topk_group: int,
                  group_topk: int, tie_eps: float) -> bool:
    E = b.size
    if len(set(sel.tolist())) != k or sel.min() < 0 or sel.max() >= E:
        return False
    if n_group <= 1:
        return _near_topk(b, sel, k, tie_eps)
    # Group-limited: the kept groups must hold every chosen expert and be a
    # top-topk_group set of group scores (each a sum of group_topk scores, so
    # its tolerance is group_topk * tie_eps); the experts must then be a
    # top-k inside the kept groups.  Groups not implied by the choice are
    # filled with the best remaining ones.
    gs = E // n_group
    gscore = moe.group_scores(b[None, :], n_group, group_topk)[0]
    used = sorted(set((sel // gs).tolist()))
    if len(used) > topk_group:
        return False
    others = [g for g in np.argsort(-gscore, kind="stable") if g not in used]
    kept = np.array(used + others[:topk_group - len(used)], dtype=np.int64)
    geps = group_topk * tie_eps
    kth_g = -np.sort(-gscore)[topk_group - 1]
    dropped = np.delete(gscore, kept)
    if gscore[kept].min() < kth_g - geps:
        return False
    if dropped.size and dropped.max() > gscore[kept].min() + geps:
        return False
    allowed = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in sorted(kept)])
    pos = {int(e): i for i, e in enumerate(allowed)}
    return _near_topk(b[allowed], np.array([pos[int(e)] for e in sel]), k, tie_eps)


def compare_routing(idx: np.ndarray, w: np.ndarray, x, router_w, corr_bias, k: int,
                    scale: float, ref: Optional[moe.Routing] = None,
                    tie_eps: float = 1e-5, n_group: int = 1, topk_group: int = 1,
                    group_topk: int = 2) -> RoutingReport:
    """Indices slot for slot against the oracle, near-ties excused (see above).

    With ``n_group`` > 1 the routing is group-limited; a differing choice is
    valid when its kept groups and its experts are both near-top choices.
    """
    idx = np.asarray(idx, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    groups = dict(n_group=n_group, topk_group=topk_group, group_topk=group_topk)
    r = ref if ref is not None else moe.route(x, router_w, corr_bias, k, scale, **groups)
    T, E = r.beta.shape
    forced = r.idx.copy()
    exact = (idx == r.idx).all(axis=1)
    invalid, excused = [], 0
    for t in np.nonzero(~exact)[0]:
        if _valid_choice(r.beta[t], idx[t], k, n_group, topk_group, group_topk, tie_eps):
            excused += 1
            forced[t] = idx[t]
        else:
            invalid.append(int(t))
    rf = moe.route(x, router_w, corr_bias, k, scale, force_idx=forced)
    good = np.ones(T, bool)
    good[invalid] = False
    max_dw = float(np.abs(w[good] - rf.weight[good]).max()) if good.any() else 0.0
    sum_err = float(np.abs(w.sum(axis=1) - scale).max()) if T else 0.0
    return RoutingReport(T, int(exact.sum()), excused, invalid, forced, max_dw, sum_err)


@dataclasses.dataclass
class OutputReport:
    rms: float
    max_rel: float    # max |out - ref| / rms(ref)
    mean_rel: float   # mean |out - ref| / rms(ref)


def compare_output(out: np.ndarray, ref: np.ndarray) -> OutputReport:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    if rms == 0.0:
        rms = 1.0
    d = np.abs(out - ref)
    return OutputReport(rms, float(d.max() / rms) if d.size else 0.0,
                        float(d.mean() / rms) if d.size else 0.0)


# Output tolerances of the layer, relative to the output RMS.
BF16_MAX_REL = 2e-2
BF16_MEAN_REL = 2e-3
F32_MAX_REL = 1e-5
WEIGHT_TOL = 1e-5
# The MXFP8 layer is held to the bf16 bounds above against oracle.forward_mx,
# which performs the same quantisations.


# ------------------------------------------------------ MXFP8 rounding ties

# Error budget of an MXFP8 dot product computed by the block-scaled FP8 MFMA,
# relative to the sum of the magnitudes of its terms, for the diagnostic
# below.  It was measured on the GPU, not derived: the MFMA sums each
# 64-element step with limited internal precision, and on gfx950 the error of
# one step reached 1.7e-5 of that sum, and 6.1e-5 over a 512-long product, for
# identical inputs; 2^-13 (1.2e-4) is the budget used here.  Because it comes
# from the hardware under test, mx_explain is a diagnostic and never the
# pass condition of a parity test.
MX_HW_REL = 2.0 ** -13


def mx_hidden_budget(xq: np.ndarray, w1, w3, eps: float = MX_HW_REL):
    """The oracle's gated hidden values h = SiLU(xq W1^T) * (xq W3^T) of an
    MXFP8 expert (``oracle.expert_hidden_mx``) and the error budget ``eh`` of a
    kernel's fp32 value of h: each product may be off by ``eps`` times the sum
    of its term magnitudes, propagated to first order through SiLU(g) * u, plus
    their product and a few fp32 roundings of the epilogue (2^-20 |h|)."""
    W1, W3 = mx.dequantize(*w1), mx.dequantize(*w3)
    h = moe.expert_hidden_mx(xq, w1, w3)
    g, u = xq @ W1.T, xq @ W3.T
    ax = np.abs(xq)
    eg, eu = eps * (ax @ np.abs(W1).T), eps * (ax @ np.abs(W3).T)
    sg = 1.0 / (1.0 + np.exp(-g))
    eh = (np.abs(sg * (1.0 + g * (1.0 - sg)) * u) * eg + np.abs(g * sg) * eu + eg * eu
          + 2.0 ** -20 * np.abs(h))
    return h, eh


@dataclasses.dataclass
class MxHiddenReport:
    values: int          # hidden values checked
    same: int            # kernel code and block scale equal to the oracle's rounding of h
    other_valid: int     # different, but the rounding of a value within the budget of h
    invalid: int         # neither
    blocks: int
    scale_other: int     # block scales different from the oracle's but valid
    scale_invalid: int


def mx_hidden_check(codes: np.ndarray, scales: np.ndarray, h: np.ndarray,
                    eh: np.ndarray) -> MxHiddenReport:
    """A kernel's MXFP8 hidden rows (E4M3 ``codes`` [n, F], E8M0 ``scales``
    [n, F/32]) against the oracle's values ``h`` with error budget ``eh``.

    The kernel takes each rounding decision once, on its own fp32 value of h.
    A decision is valid when it is the oracle's rounding rule applied to some
    value within ``eh`` of h:
      * block scale 2^s: block_exponent(a) == s for some block maximum a in
        [max(|h| - eh), max(|h| + eh)] (block_exponent is monotone);
      * element code q (value at the kernel's scale): |q - h| <= eh + half the
        E4M3 spacing at q's magnitude (the largest distance from which
        round-to-nearest lands on q).
    """
    n, F = h.shape
    nb = F // mx.BLOCK
    s_k = np.asarray(scales).astype(np.int64).reshape(n, nb) - 127
    q = mx.dequantize(codes, scales)
    oc, osc = mx.quantize(h)
    same = (np.asarray(codes) == oc) & np.repeat(np.asarray(scales).reshape(n, nb) == osc,
                                                  mx.BLOCK, axis=1)
    hb, eb = np.abs(h).reshape(n, nb, mx.BLOCK), eh.reshape(n, nb, mx.BLOCK)
    lo = np.maximum(hb - eb, 0.0).max(axis=-1)
    hi = (hb + eb).max(axis=-1)
    s_lo = np.where(lo > 0, mx.block_exponent(lo), np.iinfo(np.int64).min)
    s_hi = mx.block_exponent(hi)
    scale_ok = (s_lo <= s_k) & (s_k <= s_hi)
    sc = np.repeat(np.ldexp(1.0, s_k), mx.BLOCK, axis=1)
    y = np.abs(q) / sc
    _, x = np.frexp(np.maximum(y, 2.0 ** -6))
    half = np.ldexp(1.0, x - 1 - 3) / 2 * sc       # half the spacing of y's binade, scaled
    elem_ok = np.abs(q - h) <= eh + half
    return MxHiddenReport(int(h.size), int(same.sum()), int((~same & elem_ok).sum()),
                          int((~elem_ok).sum()), int(n * nb),
                          int((scale_ok & (s_k + 127 != osc)).sum()), int((~scale_ok).sum()))


def _e4m3_neighbours(a: np.ndarray):
    """The E4M3 grid values below and above |a| (a in [0, 448])."""
    _, x = np.frexp(np.maximum(a, 2.0 ** -6))
    step = np.ldexp(1.0, x - 1 - 3)          # spacing in a's binade (2^-9 below 2^-6)
    lo = np.floor(a / step) * step
    return lo, lo + step


@dataclasses.dataclass
class MxFlipReport:
    rms: float
    mean_rel: float        # mean |out - ref| / rms before any explanation
    candidates: int        # hidden values (or blocks) whose rounding is ambiguous
    flips: int             # candidates taken to explain the difference
    max_resid_rel: float   # max |residual| / rms after the flips
    violations: int        # outputs with |residual| > accumulation tolerance


def mx_explain(out, ref, x_in, routing: moe.Routing, experts, shared,
               eps: float = MX_HW_REL, progress=None) -> MxFlipReport:
    """Explain the difference between an MXFP8 layer output and
    ``oracle.forward_mx`` by alternative roundings that are equally correct.

    For every expert row the oracle recomputes g = xq W1^T, u = xq W3^T and
    h = SiLU(g) u, with error budgets eg = eps |xq||W1|^T (likewise eu) and
    eh = |SiLU'(g) u| eg + |SiLU(g)| eu.  A hidden value whose E4M3 rounding
    decision lies within eh of its midpoint may take the other neighbour; a
    block whose maximum lies within its budget of a scale boundary may take
    the neighbouring scale.  Each such alternative is a candidate whose effect
    on the token's output row is v = w (alternative - chosen) W2^T (w: the
    routing weight, 1 for the shared expert).  A candidate is taken when it
    reduces the squared difference: candidates with 2 <r, v> > |v|^2 against
    the token's difference r are kept, then taken greedily (largest reduction
    first, r updated) while any reduces |r|^2.  What remains must lie within the
    accumulation tolerance eps * w |hq||W2|^T (summed over the token's experts)
    + 1e-6 * rms, element by element.
    """
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    xq = mx.fake_quantize(moe.decode(x_in))
    T, D = xq.shape
    resid = out - ref
    tol = np.zeros((T, D))
    vecs = [[] for _ in range(T)]   # effects of the candidates each token might take
    count = {"cand": 0, "flips": 0}

    def slot(tok, wt, w1, w3, w2):
        rows = xq[tok]
        W1, W3, W2 = mx.dequantize(*w1), mx.dequantize(*w3), mx.dequantize(*w2)
        g, u = rows @ W1.T, rows @ W3.T
        ar = np.abs(rows)
        eg, eu = eps * (ar @ np.abs(W1).T), eps * (ar @ np.abs(W3).T)
        sg = 1.0 / (1.0 + np.exp(-g))
        h = g * sg * u
        eh = (np.abs(sg * (1.0 + g * (1.0 - sg)) * u) * eg + np.abs(g * sg) * eu
              + 2.0 ** -20 * np.abs(h))
        hq = mx.fake_quantize(h)
        tol[tok] += np.abs(wt)[:, None] * eps * (np.abs(hq) @ np.abs(W2).T)
        n, F = h.shape
        nb = F // mx.BLOCK
        hb, eb, qb = (a.reshape(n, nb, mx.BLOCK) for a in (h, eh, hq))
        amax = np.abs(hb).max(axis=-1)
        emax = np.take_along_axis(eb, np.abs(hb).argmax(axis=-1)[..., None], axis=-1)[..., 0]
        s = mx.block_exponent(amax)
        sc = np.ldexp(1.0, s)[..., None]
        y, ey = np.abs(hb) / sc, eb / sc
        lo, hi = _e4m3_neighbours(y)
        alt = np.where(np.abs(qb) / sc == lo, hi, lo)
        elem = (np.abs(y - (lo + hi) / 2) <= ey) & (hi <= mx.E4M3_MAX)
        dv = (wt[:, None, None] * np.where(elem, np.sign(hb) * (alt * sc - np.abs(qb)), 0.0)
              ).reshape(n, F)
        R = resid[tok]
        G = R @ W2                                   # <r_t, W2[:, f]>
        cn = np.einsum("df,df->f", W2, W2)           # |W2[:, f]|^2
        pre = elem.reshape(n, F) & (2 * dv * G > dv * dv * cn[None, :])
        for i, f in zip(*np.nonzero(pre)):
            vecs[tok[i]].append(dv[i, f] * W2[:, f])
        count["cand"] += int(elem.sum())
        # scale candidates: the whole block at the neighbouring scale
        for s_alt in (-1, 1):
            near = mx.block_exponent(np.maximum(amax + s_alt * emax, 0.0)) != s
            for i, b in zip(*np.nonzero(near)):
                blk = hb[i, b]
                sa = s[i, b] + s_alt
                yy = np.minimum(np.abs(blk) / 2.0 ** sa, mx.E4M3_MAX)
                alt_blk = np.sign(blk) * mx.decode_e4m3(mx.encode_e4m3(yy)) * 2.0 ** sa
                v = wt[i] * (W2[:, b * mx.BLOCK:(b + 1) * mx.BLOCK] @ (alt_blk - qb[i, b]))
                count["cand"] += 1
                if 2 * (R[i] @ v) > v @ v:
                    vecs[tok[i]].append(v)

    used_experts = np.unique(routing.idx)
    for n_done, e in enumerate(used_experts):
        tok, sl = np.nonzero(routing.idx == e)
        slot(tok, routing.weight[tok, sl], *experts(int(e)))
        if progress is not None and n_done % 32 == 31:
            progress(f"mx_explain: {n_done + 1}/{len(used_experts)} experts")
    slot(np.arange(T), np.ones(T), *shared)

    rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
    left = resid.copy()
    for t in range(T):
        if not vecs[t]:
            continue
        V = np.array(vecs[t])
        vv = np.einsum("ij,ij->i", V, V)
        used = np.zeros(len(V), bool)
        r = left[t]
        while True:  # greedy: the candidate that reduces |r|^2 most, until none does
            gain = 2 * (V @ r) - vv
            gain[used] = -np.inf
            c = int(np.argmax(gain))
            if gain[c] <= 0:
                break
            r -= V[c]
            used[c] = True
            count["flips"] += 1
    viol = int((np.abs(left) > tol + 1e-6 * rms).sum())
    return MxFlipReport(rms, float(np.abs(resid).mean() / rms), count["cand"], count["flips"],
                        float(np.abs(left).max() / rms), viol)
