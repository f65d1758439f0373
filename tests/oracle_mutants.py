"""Plausible mistakes planted in the CPU oracle, to show that the pins catch them.

Each mutant replaces one or two functions of ``oracle.moe`` (or ``oracle.mx``)
in the running process; nothing is written to disk.  ``tests/conftest.py``
applies the mutant named by the environment variable ``GLM_ORACLE_MUTANT`` at
the start of a pytest session, and ``tests/test_oracle_mutants.py`` runs the
oracle's pin files once per mutant in a child pytest process, expecting them
to fail.

The mistakes are misreadings of the layer statement (frontier-model-atlas
"GLM-5.2 model anatomy", Mixture of Experts panel; PocketLLM "GLM-5.2",
Implemented execution path for the w1/w3/w2 roles) or of the rows built next
to it (group routing, RMSNorm, MXFP8).
"""
from __future__ import annotations

import numpy as np

ENV = "GLM_ORACLE_MUTANT"


def _route(moe, *, bias_on_logit=False, weight_from_beta=False, renorm="selected",
           softmax=False, bias_sign=1.0):
    """A routing function with one of its steps misread."""

    def route(x, router_w, corr_bias, top_k, scale, force_idx=None, n_group=1, topk_group=1,
              group_topk=2):
        x = moe.decode(x)
        W = moe.decode(router_w)
        b = moe.decode(corr_bias)
        z = x @ W.T
        if softmax:
            ez = np.exp(z - z.max(axis=1, keepdims=True))
            sigma = ez / ez.sum(axis=1, keepdims=True)
        else:
            sigma = moe.sigmoid(z)
        beta = moe.sigmoid(z + b[None, :]) if bias_on_logit else sigma + bias_sign * b[None, :]
        if force_idx is None:
            idx = moe.select_topk_grouped(beta, top_k, n_group, topk_group, group_topk)
        else:
            idx = np.asarray(force_idx, dtype=np.int64)
        src = beta if weight_from_beta else sigma
        sel = np.take_along_axis(src, idx, axis=1)
        if renorm == "selected":
            weight = sel / sel.sum(axis=1, keepdims=True) * scale
        elif renorm == "all":
            weight = sel / src.sum(axis=1, keepdims=True) * scale
        else:
            weight = sel * scale
        return moe.Routing(idx=idx.astype(np.int64), weight=weight, sigma=sigma, beta=beta)

    return route


def _bias_on_logit(moe, mx):
    return moe, {"route": _route(moe, bias_on_logit=True)}


def _weights_from_beta(moe, mx):
    return moe, {"route": _route(moe, weight_from_beta=True)}


def _no_renorm(moe, mx):
    return moe, {"route": _route(moe, renorm="none")}


def _renorm_over_all_experts(moe, mx):
    return moe, {"route": _route(moe, renorm="all")}


def _softmax_router(moe, mx):
    return moe, {"route": _route(moe, softmax=True)}


def _bias_subtracted(moe, mx):
    return moe, {"route": _route(moe, bias_sign=-1.0)}


def _gate_up_swapped(moe, mx):
    orig = moe.expert_mlp

    def expert_mlp(xr, w1, w3, w2):
        return orig(xr, w3, w1, w2)

    return moe, {"expert_mlp": expert_mlp}


def _shared_scaled(moe, mx):
    orig = moe.forward

    def forward(x, router_w, corr_bias, experts, shared, top_k, scale, force_idx=None,
                routing=None, n_group=1, topk_group=1, group_topk=2):
        out, r = orig(x, router_w, corr_bias, experts, shared, top_k, scale, force_idx, routing,
                      n_group, topk_group, group_topk)
        return out + (scale - 1.0) * moe.expert_mlp(moe.decode(x), *shared), r

    return moe, {"forward": forward}


def _upper_index_ties(moe, mx):
    def select_topk(beta, k):
        E = beta.shape[-1]
        order = np.argsort(-beta[..., ::-1], axis=-1, kind="stable")
        return (E - 1 - order)[..., :k]

    return moe, {"select_topk": select_topk}


def _slots_by_index(moe, mx):
    orig = moe.select_topk

    def select_topk(beta, k):
        return np.sort(orig(beta, k), axis=-1)

    return moe, {"select_topk": select_topk}


def _sigmoid_for_silu(moe, mx):
    return moe, {"silu": lambda v: 1.0 / (1.0 + np.exp(-v))}


def _group_score_is_max(moe, mx):
    def group_scores(beta, n_group, group_topk=2):
        T, E = beta.shape
        return beta.reshape(T, n_group, E // n_group).max(axis=2)

    orig_sel = moe.select_topk

    def select_topk_grouped(beta, k, n_group, topk_group, group_topk=2):
        if n_group <= 1:
            return orig_sel(beta, k)
        T, E = beta.shape
        gs = E // n_group
        keep = np.argsort(-group_scores(beta, n_group), axis=1, kind="stable")[:, :topk_group]
        allowed = np.zeros((T, n_group), dtype=bool)
        np.put_along_axis(allowed, keep, True, axis=1)
        return orig_sel(np.where(np.repeat(allowed, gs, axis=1), beta, -np.inf), k)

    return moe, {"group_scores": group_scores, "select_topk_grouped": select_topk_grouped}


def _rmsnorm_without_eps(moe, mx):
    def rmsnorm(h, weight, eps):
        h = moe.decode(h)
        return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True)) * moe.decode(weight)

    return moe, {"rmsnorm": rmsnorm}


def _e4m3_truncates(moe, mx):
    orig = mx.encode_e4m3

    def encode_e4m3(v):
        v = np.asarray(v, dtype=np.float64)
        a = np.abs(v)
        _, x = np.frexp(a)
        step = np.ldexp(1.0, np.maximum(x - 1, -6) - 3)
        return orig(np.sign(v) * np.floor(a / step) * step)  # round toward zero

    return mx, {"encode_e4m3": encode_e4m3}


def _mx_scale_one_too_large(moe, mx):
    orig = mx.block_exponent

    def block_exponent(amax):
        return orig(amax) + 1

    return mx, {"block_exponent": block_exponent}


MUTANTS = {
    "bias_on_logit": _bias_on_logit,
    "weights_from_beta": _weights_from_beta,
    "no_renorm": _no_renorm,
    "renorm_over_all_experts": _renorm_over_all_experts,
    "softmax_router": _softmax_router,
    "bias_subtracted": _bias_subtracted,
    "gate_up_swapped": _gate_up_swapped,
    "shared_scaled": _shared_scaled,
    "upper_index_ties": _upper_index_ties,
    "slots_by_index": _slots_by_index,
    "sigmoid_for_silu": _sigmoid_for_silu,
    "group_score_is_max": _group_score_is_max,
    "rmsnorm_without_eps": _rmsnorm_without_eps,
    "e4m3_truncates": _e4m3_truncates,
    "mx_scale_one_too_large": _mx_scale_one_too_large,
}


def apply(name: str) -> None:
    """Plant mutant ``name`` in the imported oracle (module attributes and the
    package's re-exports, so both internal and external calls see it)."""
    import oracle
    from oracle import moe, mx

    target, fns = MUTANTS[name](moe, mx)
    for attr, fn in fns.items():
        setattr(target, attr, fn)
        if target is moe and hasattr(oracle, attr):
            setattr(oracle, attr, fn)
