"""The comparison rules of ``oracle.parity`` (CPU): a choice equal to the
oracle's is exact, a swap at a near-tie is excused, anything else is invalid,
with and without group-limited routing."""
import numpy as np

import oracle
from oracle import parity


def _layer(T=6, D=16, E=16, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    W = rng.standard_normal((E, D)) * 0.3
    b = rng.standard_normal(E) * 0.01
    return x, W, b


def test_oracle_choice_is_exact():
    x, W, b = _layer()
    r = oracle.route(x, W, b, 4, 2.5)
    rep = parity.compare_routing(r.idx, r.weight, x, W, b, 4, 2.5)
    assert rep.ok and rep.exact == rep.tokens and rep.excused == 0
    assert rep.max_weight_err == 0.0


def test_wrong_choice_is_invalid():
    x, W, b = _layer()
    r = oracle.route(x, W, b, 4, 2.5)
    idx = r.idx.copy()
    # replace the best expert of token 2 by the worst one
    idx[2, 0] = int(np.argmin(r.beta[2]))
    rep = parity.compare_routing(idx, r.weight, x, W, b, 4, 2.5)
    assert rep.invalid == [2]


def test_near_tie_swap_is_excused_and_forced():
    x, W, b = _layer()
    r = oracle.route(x, W, b, 4, 2.5)
    t = 1
    s = np.sort(r.beta[t])[::-1]
    fifth = int(np.argsort(-r.beta[t], kind="stable")[4])
    # move the correction bias so experts k and k+1 of token t differ by 1e-7
    b2 = b.copy()
    b2[fifth] += s[3] - s[4] - 1e-7
    r2 = oracle.route(x, W, b2, 4, 2.5)
    idx = r2.idx.copy()
    idx[t, 3] = fifth if r2.idx[t, 3] != fifth else int(np.argsort(-r2.beta[t])[4])
    rep = parity.compare_routing(idx, r2.weight, x, W, b2, 4, 2.5)
    assert rep.ok and rep.excused == 1
    np.testing.assert_array_equal(rep.forced_idx[t], idx[t])


def test_missing_or_repeated_expert_is_invalid():
    x, W, b = _layer()
    r = oracle.route(x, W, b, 4, 2.5)
    idx = r.idx.copy()
    idx[0, 1] = idx[0, 0]
    rep = parity.compare_routing(idx, r.weight, x, W, b, 4, 2.5)
    assert rep.invalid == [0]


GROUPS = dict(n_group=4, topk_group=2, group_topk=2)


def test_grouped_oracle_choice_is_exact():
    x, W, b = _layer(T=20, E=16, seed=3)
    r = oracle.route(x, W, b, 4, 1.0, **GROUPS)
    rep = parity.compare_routing(r.idx, r.weight, x, W, b, 4, 1.0, **GROUPS)
    assert rep.ok and rep.exact == rep.tokens


def test_plain_topk_is_invalid_under_groups_where_it_crosses_groups():
    x, W, b = _layer(T=40, E=16, seed=4)
    plain = oracle.route(x, W, b, 4, 1.0)
    grouped = oracle.route(x, W, b, 4, 1.0, **GROUPS)
    differ = np.nonzero((plain.idx != grouped.idx).any(axis=1))[0]
    assert differ.size > 0
    rep = parity.compare_routing(plain.idx, plain.weight, x, W, b, 4, 1.0, **GROUPS)
    assert set(rep.invalid) == set(differ.tolist())


def test_group_near_tie_swap_is_excused():
    # token 0: groups 1 and 2 tie for the second kept group up to 1e-8
    E, gs = 16, 4
    beta_target = np.full(E, 0.1)
    beta_target[0:4] = [0.9, 0.8, 0.2, 0.1]          # group 0: best
    beta_target[4:8] = [0.6, 0.5, 0.1, 0.1]          # group 1: 1.1
    beta_target[8:12] = [0.7, 0.4 + 1e-8, 0.1, 0.1]  # group 2: 1.1 + 1e-8
    D = E
    x = np.ones((1, D))
    # sigma = beta - b; choose b = 0 and a router that yields logit(beta)
    z = np.log(beta_target / (1 - beta_target))
    W = np.diag(z)
    b = np.zeros(E)
    r = oracle.route(x, W, b, 4, 1.0, **GROUPS)
    assert set((r.idx[0] // gs).tolist()) == {0, 2}
    other = np.array([[0, 1, 4, 5]])   # groups 0 and 1 instead
    rep = parity.compare_routing(other, r.weight, x, W, b, 4, 1.0, **GROUPS)
    assert rep.ok and rep.excused == 1
    # the same swap with a clear gap is invalid
    beta_target[9] = 0.45
    W = np.diag(np.log(beta_target / (1 - beta_target)))
    rep = parity.compare_routing(other, r.weight, x, W, b, 4, 1.0, **GROUPS)
    assert rep.invalid == [0]


# ------------------------------------------------------- MXFP8 rounding ties

from oracle import mx  # noqa: E402


def test_compare_output_hand_values():
    """max and mean |out - ref| relative to rms(ref), on values worked by hand.

    ref = [[3, -4], [0, 0]]: rms = sqrt((9 + 16) / 4) = 2.5.  out differs by
    +0.5 at (0, 0) and -0.25 at (1, 1): max 0.5 / 2.5 = 0.2, mean
    0.75 / 4 / 2.5 = 0.075 (the sign of a difference does not matter).
    """
    ref = np.array([[3.0, -4.0], [0.0, 0.0]])
    out = np.array([[3.5, -4.0], [0.0, -0.25]])
    o = parity.compare_output(out, ref)
    assert o.rms == 2.5
    assert o.max_rel == 0.2
    assert o.mean_rel == 0.075
    # swapping the roles changes the rms (out is not the reference)
    assert parity.compare_output(ref, out).rms != 2.5
    # an all-zero reference: differences are absolute
    z = parity.compare_output(np.array([0.5, -1.0]), np.zeros(2))
    assert (z.rms, z.max_rel, z.mean_rel) == (1.0, 1.0, 0.75)
    # float32 inputs are compared in float64
    o32 = parity.compare_output(out.astype(np.float32), ref.astype(np.float32))
    assert (o32.max_rel, o32.mean_rel) == (0.2, 0.075)


def _mx_layer(seed=9, T=48, D=256, E=8, F=128, k=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    W = rng.standard_normal((E, D)) * 0.1
    b = rng.standard_normal(E) * 0.01
    q = lambda a: mx.quantize(a)
    ex = {e: (q(rng.standard_normal((F, D)) / 16), q(rng.standard_normal((F, D)) / 16),
              q(rng.standard_normal((D, F)) / 11)) for e in range(E)}
    sh = (q(rng.standard_normal((F, D)) / 16), q(rng.standard_normal((F, D)) / 16),
          q(rng.standard_normal((D, F)) / 11))
    return x, W, b, ex, sh, k


def _fp32_mx_layer(x, r, ex, sh):
    """The MXFP8 layer with the expert products in fp32 (a stand-in for a GPU
    result: same quantisation rules, hidden values rounded from fp32)."""
    xq = mx.fake_quantize(x).astype(np.float32)
    def mlp(rows, w1, w3, w2):
        W1, W3, W2 = (mx.dequantize(*w).astype(np.float32) for w in (w1, w3, w2))
        g, u = rows @ W1.T, rows @ W3.T
        h = (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float32)
        return mx.fake_quantize(h.astype(np.float64)) @ W2.T.astype(np.float64)
    out = np.zeros(x.shape)
    for e in np.unique(r.idx):
        tok, slot = np.nonzero(r.idx == e)
        out[tok] += r.weight[tok, slot][:, None] * mlp(xq[tok], *ex[e])
    return out + mlp(xq, *sh)


def _layer_from_hidden(x, r, ex, sh, edit=None):
    """The MXFP8 layer evaluated with the oracle's numbers, except that
    ``edit(slot_key, hq)`` may change the quantised hidden rows of a slot."""
    xq = mx.fake_quantize(x)
    def mlp(key, rows, w1, w3, w2):
        W1, W3, W2 = (mx.dequantize(*w) for w in (w1, w3, w2))
        h = (lambda g, u: g / (1 + np.exp(-g)) * u)(rows @ W1.T, rows @ W3.T)
        hq = mx.fake_quantize(h)
        if edit is not None:
            hq = edit(key, h, hq)
        return hq @ W2.T
    out = np.zeros(x.shape)
    for e in np.unique(r.idx):
        tok, slot = np.nonzero(r.idx == e)
        out[tok] += r.weight[tok, slot][:, None] * mlp(int(e), xq[tok], *ex[e])
    return out + mlp("shared", xq, *sh)


def test_mx_explain_accepts_equal_and_fp32_results():
    x, W, b, ex, sh, k = _mx_layer()
    ref, r = oracle.forward_mx(x, W, b, lambda e: ex[e], sh, k, 2.5)
    same = parity.mx_explain(ref, ref, x, r, lambda e: ex[e], sh)
    assert same.violations == 0 and same.flips == 0 and same.mean_rel == 0
    got = _fp32_mx_layer(x, r, ex, sh)
    rep = parity.mx_explain(got, ref, x, r, lambda e: ex[e], sh)
    assert rep.violations == 0, rep


def _midpoint_element(h, hq):
    """(row, col) of the hidden value closest (relatively) to an E4M3 midpoint,
    and the value with its rounding moved to the other neighbour."""
    n, F = h.shape
    s = mx.block_exponent(np.abs(h.reshape(n, F // 32, 32)).max(-1)).repeat(32, axis=1)
    y = np.abs(h) / np.exp2(s)
    lo, hi = parity._e4m3_neighbours(y)
    dist = np.abs(y - (lo + hi) / 2) / (hi - lo)
    dist[np.abs(h) == np.abs(h.reshape(n, F // 32, 32)).max(-1).repeat(32, axis=1)] = np.inf
    i, f = np.unravel_index(np.argmin(dist), dist.shape)
    chosen = np.abs(hq[i, f]) / 2.0 ** s[i, f]
    alt = hi[i, f] if chosen == lo[i, f] else lo[i, f]
    return i, f, np.sign(h[i, f]) * alt * 2.0 ** s[i, f], dist[i, f]


def test_mx_explain_takes_a_flip_at_a_midpoint_and_nothing_else():
    x, W, b, ex, sh, k = _mx_layer(seed=11)
    ref, r = oracle.forward_mx(x, W, b, lambda e: ex[e], sh, k, 2.5)
    picked = {}

    def flip_near(key, h, hq):
        if key != "shared":
            return hq
        i, f, v, dist = _midpoint_element(h, hq)
        picked["dist"] = dist
        hq = hq.copy()
        hq[i, f] = v
        return hq

    got = _layer_from_hidden(x, r, ex, sh, flip_near)
    rep = parity.mx_explain(got, ref, x, r, lambda e: ex[e], sh)
    assert picked["dist"] < 1e-3
    assert rep.violations == 0 and rep.flips == 1, rep

    def flip_far(key, h, hq):
        if key != "shared":
            return hq
        hq = hq.copy()
        # the rounding of a value far from any midpoint moved by one step
        n, F = h.shape
        s = mx.block_exponent(np.abs(h.reshape(n, F // 32, 32)).max(-1)).repeat(32, axis=1)
        y = np.abs(h) / np.exp2(s)
        lo, hi = parity._e4m3_neighbours(y)
        dist = np.abs(y - (lo + hi) / 2) / (hi - lo)
        i, f = np.unravel_index(np.argmax(np.where(np.abs(h) > 0.1, dist, -1)), dist.shape)
        hq[i, f] += np.sign(h[i, f]) * (hi[i, f] - lo[i, f]) * 2.0 ** s[i, f]
        return hq

    bad = _layer_from_hidden(x, r, ex, sh, flip_far)
    assert parity.mx_explain(bad, ref, x, r, lambda e: ex[e], sh).violations > 0


def test_mx_explain_flags_small_output_errors():
    x, W, b, ex, sh, k = _mx_layer(seed=12)
    ref, r = oracle.forward_mx(x, W, b, lambda e: ex[e], sh, k, 2.5)
    bad = ref.copy()
    rms = np.sqrt((ref ** 2).mean())
    bad[3, 7] += 1e-2 * rms
    assert parity.mx_explain(bad, ref, x, r, lambda e: ex[e], sh).violations == 1


# --------------------------------------------- MXFP8 hidden-value decisions

def _mx_hidden(seed=3, n=6, F=128):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, F)) * np.exp(rng.normal(0, 1, (n, 1)))
    codes, scales = oracle.mx.quantize(h)
    return h, codes, scales


def test_mx_hidden_check_accepts_the_oracle_rounding():
    h, codes, scales = _mx_hidden()
    rep = parity.mx_hidden_check(codes, scales, h, 1e-9 * np.abs(h))
    assert rep.same == rep.values == h.size
    assert rep.invalid == rep.other_valid == rep.scale_invalid == rep.scale_other == 0


def test_mx_hidden_check_takes_a_flip_at_a_midpoint_only_within_budget():
    h, codes, scales = _mx_hidden()
    mx = oracle.mx
    # move element (2, 5) onto the midpoint between its code and the next one up
    s = np.ldexp(1.0, scales[2, 0].astype(np.int64) - 127)
    y = abs(h[2, 5]) / s
    lo_code = mx.encode_e4m3(np.array([y]))[0]
    v0 = mx.decode_e4m3(np.array([lo_code]))[0]
    nxt = mx.decode_e4m3(np.array([lo_code + 1]))[0]
    h[2, 5] = np.sign(h[2, 5]) * (v0 + nxt) / 2 * s * (1 - 1e-9)  # just below the midpoint
    codes, scales = mx.quantize(h)
    flipped = codes.copy()
    flipped[2, 5] = codes[2, 5] + 1 if mx.decode_e4m3(codes[2, 5:6])[0] == np.sign(h[2, 5]) * v0 \
        else codes[2, 5] - 1
    eh = 1e-6 * np.abs(h)
    rep = parity.mx_hidden_check(flipped, scales, h, eh)
    assert (rep.same, rep.other_valid, rep.invalid) == (h.size - 1, 1, 0)
    # the same flip two codes away is not a rounding of any value in budget
    far = codes.copy()
    far[2, 5] = flipped[2, 5] + (flipped[2, 5].astype(int) - codes[2, 5].astype(int))
    assert parity.mx_hidden_check(far, scales, h, eh).invalid == 1


def test_mx_hidden_check_rejects_a_wrong_scale_and_a_permuted_row():
    h, codes, scales = _mx_hidden()
    bad = scales.copy()
    bad[1, 2] += 1   # one binade too coarse: within range, but not the rule's choice
    rep = parity.mx_hidden_check(codes, bad, h, 1e-9 * np.abs(h))
    assert rep.scale_invalid == 1 and rep.invalid > 0
    # rows swapped (an indexing mistake): almost every value is invalid
    rep = parity.mx_hidden_check(codes[::-1].copy(), scales[::-1].copy(), h, 1e-6 * np.abs(h))
    assert rep.invalid > 0.8 * h.size
