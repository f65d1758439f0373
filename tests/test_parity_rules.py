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
