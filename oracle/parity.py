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

from . import moe


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
