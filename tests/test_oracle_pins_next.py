"""Pins of the oracle's group-limited routing, RMSNorm block and dense FFN (CPU).

Group routing is a GLM-4.5 feature ("Full Forward" note, How it works: sigmoid
group routing); the pre-norm block and the leading dense feed-forward layers
come from the same note and the GLM-5.2 anatomy page (Token path: 75 MoE and
3 dense FFN blocks).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ groups

def test_group_routing_hand_fixture():
    g = json.load(open(os.path.join(GOLDEN, "hand_group_routing.json")))
    beta = np.array([g["beta"]])
    np.testing.assert_allclose(oracle.group_scores(beta, g["n_group"], g["group_topk"])[0],
                               g["group_scores"], rtol=0, atol=1e-15)
    got = oracle.select_topk_grouped(beta, g["k"], g["n_group"], g["topk_group"], g["group_topk"])
    assert got[0].tolist() == g["idx"]
    assert oracle.select_topk(beta, g["k"])[0].tolist() == g["plain_idx"]


def _brute_grouped(beta, k, n_group, topk_group, group_topk):
    E = len(beta)
    gs = E // n_group
    score = [sum(sorted(beta[g * gs:(g + 1) * gs], reverse=True)[:group_topk])
             for g in range(n_group)]
    best, keep = None, None
    for sub in itertools.combinations(range(n_group), topk_group):  # lexicographic
        s = tuple(sorted((score[g] for g in sub), reverse=True))
        if best is None or s > best:
            best, keep = s, sub
    allowed = [e for e in range(E) if e // gs in keep]
    # rank inside the kept groups: higher score, then lower index
    sel = sorted(allowed, key=lambda e: (-beta[e], e))[:k]
    return sel


@pytest.mark.parametrize("n_group,topk_group,k", [(4, 2, 2), (4, 1, 2), (2, 1, 3), (8, 3, 4)])
def test_group_routing_brute_force(n_group, topk_group, k):
    rng = np.random.default_rng(100 + n_group * 10 + topk_group)
    E = 16
    for _ in range(150):
        beta = rng.integers(0, 7, E).astype(np.float64) / 8.0 + rng.normal(0, 1e-3, E)
        got = oracle.select_topk_grouped(beta[None, :], k, n_group, topk_group)[0].tolist()
        assert got == _brute_grouped(beta.tolist(), k, n_group, topk_group, 2)


def test_grouping_that_keeps_every_group_is_plain_topk():
    w = wl.WORKLOADS["mid_bf16"]
    x, W, b = wl.make_x(w), wl.make_router_w(w), wl.make_corr_bias(w)
    plain = oracle.route(x, W, b, w.k, w.scale)
    for ng in (1, 4, 8):
        r = oracle.route(x, W, b, w.k, w.scale, n_group=ng, topk_group=ng)
        np.testing.assert_array_equal(r.idx, plain.idx)
        np.testing.assert_array_equal(r.weight, plain.weight)


def test_grouped_selection_stays_in_kept_groups_and_weights_sum_to_scale():
    w = wl.WORKLOADS["mid_bf16"]
    x, W, b = wl.make_x(w), wl.make_router_w(w), wl.make_corr_bias(w)
    r = oracle.route(x, W, b, w.k, 1.0, n_group=8, topk_group=2)
    gs = oracle.group_scores(r.beta, 8)
    kept = np.argsort(-gs, axis=1, kind="stable")[:, :2]
    assert all(set((r.idx[t] // (w.E // 8)).tolist()) <= set(kept[t].tolist()) for t in range(w.T))
    assert np.abs(r.weight.sum(1) - 1.0).max() <= 1e-12  # scale 1.0 (GLM-4.5-Air)
    plain = oracle.route(x, W, b, w.k, 1.0)
    assert (r.idx != plain.idx).any()


# ----------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_closed_form():
    eps = 1e-5
    for c in (3.0, -0.25, 1e-3):
        h = np.full((1, 16), c)
        w = np.linspace(0.5, 2.0, 16)
        want = c / math.sqrt(c * c + eps) * w
        np.testing.assert_allclose(oracle.rmsnorm(h, w, eps)[0], want, rtol=1e-15)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(3)
    h = rng.normal(0, 3, (5, 64))
    y = oracle.rmsnorm(h, np.ones(64), 0.0)
    np.testing.assert_allclose((y * y).mean(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * h, np.ones(64), 0.0), y, rtol=1e-14)


def test_round_bf16_matches_input_encoder():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e-3, 500), rng.normal(0, 1e3, 500)])
    v32 = v.astype(np.float32)
    enc = (wl.f32_to_bf16_bits(v32).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(v32.astype(np.float64)), enc)


def test_block_with_zero_ffn_is_the_residual():
    rng = np.random.default_rng(5)
    h = rng.normal(0, 1, (6, 32))
    out, _ = oracle.block_ffn(h, np.ones(32), 1e-5, "bf16", lambda x: (np.zeros_like(x), None))
    np.testing.assert_array_equal(out, h)


def test_block_passes_the_bf16_normalised_input():
    rng = np.random.default_rng(6)
    h = rng.normal(0, 2, (4, 32))
    seen = {}
    def layer(x):
        seen["x"] = x
        return x * 0, None
    oracle.block_ffn(h, np.ones(32), 1e-5, "bf16", layer)
    np.testing.assert_array_equal(seen["x"], oracle.round_bf16(oracle.rmsnorm(h, np.ones(32), 1e-5)))


# ----------------------------------------------------------- dense FFN

def test_dense_ffn_identity_closed_form():
    T, D, F = 5, 12, 6
    rng = np.random.default_rng(7)
    x = rng.normal(0, 1, (T, D))
    S = np.zeros((F, D)); S[np.arange(F), np.arange(F)] = 1.0
    Q = np.zeros((D, F)); Q[np.arange(F) + 3, np.arange(F)] = 1.0
    out = oracle.dense_ffn(x, S, 2.0 * S, Q)
    want = np.zeros((T, D))
    for t in range(T):
        for f in range(F):
            want[t, f + 3] = x[t, f] / (1.0 + math.exp(-x[t, f])) * 2.0 * x[t, f]
    np.testing.assert_allclose(out, want, rtol=1e-14, atol=1e-15)


def test_dense_ffn_equals_shared_only_layer():
    L = wl.make_layer(wl.WORKLOADS["tiny_f32"], threads=2)
    shared_only, _ = oracle.forward_arrays(L.x, L.router_w, L.corr_bias, L.w1, L.w3, L.w2,
                                           L.sw1, L.sw3, L.sw2, L.w.k, 0.0)
    np.testing.assert_allclose(oracle.dense_ffn(L.x, L.sw1, L.sw3, L.sw2), shared_only,
                               rtol=1e-13, atol=1e-14)
