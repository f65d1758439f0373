"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Every expected value here is derived independently of ``oracle.moe``: hand
fractions, brute force over subsets, closed forms of special weights, or
invariances of the layer statement (frontier-model-atlas "GLM-5.2 model
anatomy", Feed-forward / Mixture of Experts panel).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import loops
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac(s):
    return float(Fraction(s))


def _tiny(T=64, seed=1, **kw):
    w = wl.WORKLOADS["tiny_f32"].with_(T=T, seed=seed, **kw)
    return wl.make_layer(w, threads=2)


def _fwd(L, k=None, scale=None, **kw):
    w = L.w
    return oracle.forward_arrays(L.x, L.router_w, L.corr_bias, L.w1, L.w3, L.w2,
                                 L.sw1, L.sw3, L.sw2, w.k if k is None else k,
                                 w.scale if scale is None else scale, **kw)


# ------------------------------------------------------------------ spec

def test_glm_constants_match_pages():
    spec = json.load(open(os.path.join(GOLDEN, "glm52_moe_spec.json")))
    for name in ("glm_decode", "glm_prefill", "glm_skew", "glm_skew_mild"):
        w = wl.WORKLOADS[name]
        assert w.D == spec["hidden_size"]["value"]
        assert w.E == spec["routed_experts"]["value"]
        assert w.k == spec["active_experts"]["value"]
        assert w.F == spec["expert_width"]["value"]
        assert w.Fs == spec["expert_width"]["value"]  # shared width: reading, see header
        assert w.scale == spec["routed_scale"]["value"]


# ---------------------------------------------------- hand-worked routing

def test_hand_routing_fixture():
    g = json.load(open(os.path.join(GOLDEN, "hand_routing.json")))
    W = np.array([[math.log(v)] for v in g["router_w_ln"]])
    b = np.array(g["corr_bias"])
    for c in g["cases"]:
        x = np.array([[c["x"]]])
        r = oracle.route(x, W, b, c["k"], g["scale"])
        np.testing.assert_allclose(r.sigma[0], [_frac(s) for s in c["sigma"]], rtol=0, atol=1e-15)
        np.testing.assert_allclose(r.beta[0], [_frac(s) for s in c["beta"]], rtol=0, atol=1e-15)
        assert r.idx[0].tolist() == c["idx"]
        np.testing.assert_allclose(r.weight[0], [_frac(s) for s in c["weight"]], rtol=0, atol=1e-14)


# -------------------------------------------------------------- P-a: sum

@pytest.mark.parametrize("name", ["tiny_f32", "mid_bf16"])
def test_weights_sum_to_scale(name):
    w = wl.WORKLOADS[name]
    x, W, b = wl.make_x(w), wl.make_router_w(w), wl.make_corr_bias(w)
    r = oracle.route(x, W, b, w.k, w.scale)
    assert np.max(np.abs(r.weight.sum(1) - 2.5)) <= 1e-12
    assert (r.weight > 0).all()


def test_k1_weight_is_exactly_scale():
    w = wl.WORKLOADS["mid_bf16"]
    r = oracle.route(wl.make_x(w), wl.make_router_w(w), wl.make_corr_bias(w), 1, 2.5)
    assert (r.weight == 2.5).all()


# ------------------------------------------- P-b: bias selects, not weighs

def test_large_bias_forces_set_and_weights_use_unbiased_scores():
    w = wl.WORKLOADS["tiny_f32"]
    x, W = oracle.decode(wl.make_x(w)), wl.make_router_w(w).astype(np.float64)
    S = [6, 1]  # forced set, bias larger on 6 so slot order is (6, 1)
    b = np.zeros(w.E)
    b[6], b[1] = 20.0, 10.0
    r = oracle.route(x, W, b, 2, 2.5)
    assert (r.idx == np.array(S)).all()
    # independent sigmoid of an independent dot product, per token
    for t in range(x.shape[0]):
        s = [1.0 / (1.0 + math.exp(-float(np.dot(x[t], W[e])))) for e in S]
        want = [2.5 * v / sum(s) for v in s]
        np.testing.assert_allclose(r.weight[t], want, rtol=1e-13)
        # bias values do not appear in the weights
        assert not np.allclose(r.weight[t], [2.5 * (s[0] + 20) / (sum(s) + 30),
                                             2.5 * (s[1] + 10) / (sum(s) + 30)])


def test_unchanged_selection_has_identical_weights():
    w = wl.WORKLOADS["tiny_f32"]
    x, W, b = wl.make_x(w), wl.make_router_w(w), wl.make_corr_bias(w)
    r_b = oracle.route(x, W, b, w.k, w.scale)
    r_0 = oracle.route(x, W, np.zeros_like(b), w.k, w.scale)
    same = (np.sort(r_b.idx, 1) == np.sort(r_0.idx, 1)).all(1)
    diff = ~same
    assert same.sum() > 5 and diff.sum() > 0  # the bias does move some selections
    for t in np.nonzero(same)[0]:
        wb = dict(zip(r_b.idx[t], r_b.weight[t]))
        w0 = dict(zip(r_0.idx[t], r_0.weight[t]))
        for e in wb:
            assert wb[e] == w0[e]


def test_k_equals_e_ignores_bias():
    w = wl.WORKLOADS["tiny_f32"]
    x, W = oracle.decode(wl.make_x(w)), wl.make_router_w(w).astype(np.float64)
    rng = np.random.default_rng(7)
    for b in (np.zeros(w.E), rng.normal(0, 3, w.E)):
        r = oracle.route(x, W, b, w.E, 2.5)
        full = np.zeros((x.shape[0], w.E))
        np.put_along_axis(full, r.idx, r.weight, axis=1)
        sig = np.array([[1.0 / (1.0 + math.exp(-float(np.dot(x[t], W[e])))) for e in range(w.E)]
                        for t in range(x.shape[0])])
        np.testing.assert_allclose(full, 2.5 * sig / sig.sum(1, keepdims=True), rtol=1e-13)


# ---------------------------------------------- P-c: brute-force top-k

def _brute_topk(beta, k):
    """Subset with the largest sum of scores; ties: lexicographically smallest set.

    Returned in slot order: descending score, ties ascending index.
    """
    E = len(beta)
    best, best_set = None, None
    for sub in itertools.combinations(range(E), k):  # lexicographic order
        s = sum(beta[i] for i in sub)
        if best is None or s > best:
            best, best_set = s, sub
    return sorted(best_set, key=lambda e: (-beta[e], e))


def _rank_select(beta, k):
    """e is selected iff fewer than k experts beat it (higher score, or equal and lower index)."""
    E = len(beta)
    sel = [e for e in range(E)
           if sum(1 for f in range(E) if beta[f] > beta[e] or (beta[f] == beta[e] and f < e)) < k]
    return sorted(sel, key=lambda e: (-beta[e], e))


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_topk_brute_force(k):
    rng = np.random.default_rng(11 + k)
    E = 8
    for trial in range(200):
        # coarse grid of values creates many exact ties
        beta = rng.integers(0, 5, E).astype(np.float64) / 4.0
        got = oracle.select_topk(beta[None, :], k)[0].tolist()
        assert got == _rank_select(beta, k)
        assert sorted(got) == sorted(_brute_topk(beta, k)) or \
            sum(beta[got]) == sum(beta[_brute_topk(beta, k)])


def test_exact_tie_from_duplicated_router_row_goes_to_lower_index():
    w = wl.WORKLOADS["tiny_f32"]
    x = oracle.decode(wl.make_x(w))
    W = wl.make_router_w(w).astype(np.float64)
    b = wl.make_corr_bias(w).astype(np.float64)
    W[5] = W[2]
    b[5] = b[2]
    b[2] += 10.0
    b[5] += 10.0  # experts 2 and 5 bit-identical and always on top
    r = oracle.route(x, W, b, 1, 2.5)
    assert (r.idx[:, 0] == 2).all()
    r = oracle.route(x, W, b, 2, 2.5)
    assert (r.idx == np.array([2, 5])).all()


def test_topk_gap():
    beta = np.array([[0.9, 0.1, 0.5, 0.4]])
    assert oracle.topk_gap(beta, 2)[0] == pytest.approx(0.1)
    assert np.isinf(oracle.topk_gap(beta, 4)[0])


# ------------------------------- P-d: identity-like experts closed form

def _identity_layer(T, D, E, F, k, cs, ce, a, bb, seed=3, perm=None):
    """Experts with w1 = a*S, w3 = bb*S, w2 = c_e * Q (S picks the first F features,
    Q places feature f at output row perm[f])."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    W = rng.standard_normal((E, D)) / np.sqrt(D)
    bias = rng.normal(0, 0.1, E)
    perm = np.arange(F) if perm is None else perm
    S = np.zeros((F, D))
    S[np.arange(F), np.arange(F)] = 1.0
    Q = np.zeros((D, F))
    Q[perm, np.arange(F)] = 1.0
    w1 = np.stack([a * S] * E)
    w3 = np.stack([bb * S] * E)
    w2 = np.stack([c * Q for c in ce])
    return x, W, bias, w1, w3, w2, a * S, bb * S, cs * Q, perm


def _silu(v):
    return v / (1.0 + math.exp(-v))


@pytest.mark.parametrize("weights", ["ones", "per_expert"])
def test_identity_experts_closed_form(weights):
    T, D, E, F, k = 16, 24, 6, 8, 2
    ce = [1.0] * E if weights == "ones" else [float(e + 1) for e in range(E)]
    perm = np.random.default_rng(5).permutation(D)[:F]
    x, W, b, w1, w3, w2, sw1, sw3, sw2, perm = _identity_layer(
        T, D, E, F, k, cs=1.0, ce=ce, a=1.0, bb=2.0, perm=perm)
    out, r = oracle.forward_arrays(x, W, b, w1, w3, w2, sw1, sw3, sw2, k, 2.5)
    for t in range(T):
        coef = sum(r.weight[t, j] * ce[r.idx[t, j]] for j in range(k)) + 1.0
        want = np.zeros(D)
        for f in range(F):
            want[perm[f]] = coef * _silu(1.0 * x[t, f]) * (2.0 * x[t, f])
        np.testing.assert_allclose(out[t], want, rtol=1e-12, atol=1e-13)
        if weights == "ones":
            np.testing.assert_allclose(coef, 3.5, rtol=1e-13)


def test_gate_and_up_roles_are_distinct():
    """With w1 = a*S and w3 = b*S, swapping the roles would give SiLU(b x) * a x."""
    T, D, E, F, k = 4, 16, 4, 4, 1
    x, W, b, w1, w3, w2, sw1, sw3, sw2, perm = _identity_layer(
        T, D, E, F, k, cs=0.0, ce=[1.0] * E, a=1.0, bb=3.0)
    out, _ = oracle.forward_arrays(x, W, b, w1, w3, w2, sw1, sw3, sw2, k, 2.5)
    want = np.array([[2.5 * _silu(x[t, f]) * 3.0 * x[t, f] for f in range(F)] for t in range(T)])
    np.testing.assert_allclose(out[:, :F], want, rtol=1e-12)
    swapped = np.array([[2.5 * _silu(3.0 * x[t, f]) * x[t, f] for f in range(F)] for t in range(T)])
    assert not np.allclose(out[:, :F], swapped)


# ------------------------------------------------------ P-e: shared only

def _textbook_shared(x, sw1, sw3, sw2):
    g = np.einsum("td,fd->tf", x, sw1)
    u = np.einsum("td,fd->tf", x, sw3)
    h = g * (1.0 / (1.0 + np.exp(-g))) * u
    return np.einsum("tf,df->td", h, sw2)


def test_scale_zero_is_shared_expert_only():
    L = _tiny()
    out0, _ = _fwd(L, scale=0.0)
    x = L.x.astype(np.float64)
    want = _textbook_shared(x, L.sw1.astype(np.float64), L.sw3.astype(np.float64),
                            L.sw2.astype(np.float64))
    np.testing.assert_allclose(out0, want, rtol=1e-12, atol=1e-12)
    # equal to a run whose routed down projections are zero
    L2 = _tiny()
    L2.w2[:] = 0
    outz, _ = _fwd(L2)
    np.testing.assert_array_equal(out0, outz)


# ---------------------------------------------- P-f: structural invariants

def test_token_permutation_equivariance():
    L = _tiny()
    out, _ = _fwd(L)
    p = np.random.default_rng(9).permutation(L.x.shape[0])
    L.x = L.x[p]
    outp, _ = _fwd(L)
    np.testing.assert_allclose(outp, out[p], rtol=1e-12, atol=1e-13)


def test_batch_independence():
    L = _tiny()
    out, _ = _fwd(L)
    x = L.x
    L.x = x[:32]
    a, _ = _fwd(L)
    L.x = x[32:]
    b, _ = _fwd(L)
    np.testing.assert_allclose(np.concatenate([a, b]), out, rtol=1e-12, atol=1e-13)


def test_expert_relabelling_invariance():
    L = _tiny()
    out, r = _fwd(L)
    gap = oracle.topk_gap(r.beta, L.w.k)
    p = np.random.default_rng(4).permutation(L.w.E)
    L.router_w, L.corr_bias = L.router_w[p], L.corr_bias[p]
    L.w1, L.w3, L.w2 = L.w1[p], L.w3[p], L.w2[p]
    outp, rp = _fwd(L)
    ok = gap > 1e-9
    np.testing.assert_allclose(outp[ok], out[ok], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(p[rp.idx[ok]], r.idx[ok])


def test_routed_part_linear_in_w2():
    L = _tiny()
    base, _ = _fwd(L)
    shared, _ = _fwd(L, scale=0.0)
    L.w2 = L.w2 * np.float32(4.0)  # a power of two: the scaled weights are exact
    scaled, _ = _fwd(L)
    np.testing.assert_allclose(scaled - shared, 4.0 * (base - shared), rtol=1e-11, atol=1e-12)


# ------------------------------------------ P-g: scalar re-evaluation

def test_oracle_matches_scalar_loops():
    L = _tiny(T=8)
    out, r = _fwd(L)
    tolist = lambda a: a.astype(np.float64).tolist()
    for t in range(8):
        idx, wts, row = loops.layer_token(
            tolist(L.x[t]), tolist(L.router_w), tolist(L.corr_bias),
            tolist(L.w1), tolist(L.w3), tolist(L.w2),
            tolist(L.sw1), tolist(L.sw3), tolist(L.sw2), L.w.k, L.w.scale)
        assert idx == r.idx[t].tolist()
        np.testing.assert_allclose(wts, r.weight[t], rtol=1e-13)
        np.testing.assert_allclose(row, out[t], rtol=1e-11, atol=1e-12)


# ------------------------------------------------------- bf16 decoding

def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    want = [1.0, -1.0, 3.140625, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41]
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), want)
