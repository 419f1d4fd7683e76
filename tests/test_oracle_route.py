"""Pins of the oracle's routing against hand-derived values, brute force and invariants."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from workloads.inputs import make_scores, rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- hand-derived example
def test_worked_example_group_topr2():
    g = _load("route_worked_example.json")
    s = np.array(g["scores"], np.float32)
    b = np.array(g["bias"], np.float32)
    idx, w = oracle.route(s, b, g["G"], g["M"], g["k"], 2, g["route_scale"])
    assert idx.tolist() == g["r2"]["idx"]
    exp = np.array(g["r2"]["w_num"], np.float64) / np.array(g["r2"]["w_den"], np.float64)[:, None]
    np.testing.assert_allclose(w, exp, rtol=1e-15, atol=0)


def test_worked_example_bias_changes_selection():
    g = _load("route_worked_example.json")
    s = np.array(g["scores"], np.float32)
    idx, _ = oracle.route(s, np.zeros(8, np.float32), g["G"], g["M"], g["k"], 2, 1.0)
    assert idx[0].tolist() == g["r2_no_bias_token0_idx"]


def test_worked_example_group_topr1():
    g = _load("route_worked_example.json")
    s = np.array(g["scores"], np.float32)
    b = np.array(g["bias"], np.float32)
    idx, w = oracle.route(s, b, g["G"], g["M"], g["k"], 1, 1.0)
    r1 = g["r1_token0"]
    assert idx[0].tolist() == r1["idx"]
    np.testing.assert_allclose(w[0], np.array(r1["w_num"]) / r1["w_den"], rtol=1e-15)


# ---------------------------------------------------------------- brute force (two-stage definition)
def _dyadic_tie_free(seed, T, E, G, r):
    """Scores and bias on a 2^-12 grid, redrawn until no two experts of a token and
    no two group sums of a token are equal (so the optimum subsets are unique)."""
    g = rng(seed, 99, T, E)
    gsz = E // G
    while True:
        s = (g.integers(1, 4096, (T, E)) / 4096.0).astype(np.float32)
        b = (g.integers(-128, 128, E) / 4096.0).astype(np.float32)
        q = (s + b).astype(np.float64)
        ok = all(len(set(row)) == E for row in q)
        gsums = -np.sort(-q.reshape(T, G, gsz), axis=2)[:, :, :r].sum(axis=2)
        ok = ok and all(len(set(row)) == G for row in gsums)
        if ok:
            return s, b


def _brute_force(q_row, G, M, k, r):
    E = len(q_row)
    gsz = E // G
    # group score by enumeration: best sum of r members of the group
    gscore = [max(sum(c) for c in itertools.combinations(q_row[g * gsz:(g + 1) * gsz], r))
              for g in range(G)]
    best_groups = max(itertools.combinations(range(G), M), key=lambda gs: sum(gscore[x] for x in gs))
    allowed = [e for e in range(E) if e // gsz in best_groups]
    best = max(itertools.combinations(allowed, k), key=lambda es: sum(q_row[e] for e in es))
    return sorted(best, key=lambda e: (-q_row[e], e))


@pytest.mark.parametrize("E,G,M,k,r", [(16, 4, 2, 4, 2), (8, 4, 2, 3, 2), (12, 3, 2, 5, 3),
                                        (16, 8, 3, 4, 1), (16, 4, 4, 4, 2), (12, 4, 1, 2, 2)])
def test_brute_force_tiny(E, G, M, k, r):
    T = 40
    s, b = _dyadic_tie_free(E * 100 + G * 10 + M, T, E, G, r)
    idx, w = oracle.route(s, b, G, M, k, r, 1.0)
    q = (s + b).astype(np.float64)
    for t in range(T):
        assert idx[t].tolist() == _brute_force(list(q[t]), G, M, k, r)


def test_two_stage_is_not_the_joint_optimum():
    """E/G=4, k=4, M=2, r=2: the group stage keeps B and C (top-2 sums 1.25 and
    1.1875 beat A's 1.125), so all of B is selected although A's 1.0 plus three
    of B would give a larger total (2.875 against 2.5)."""
    A = [1.0, 0.125, 0.125, 0.125]
    B = [0.625] * 4
    C = [0.59375] * 4
    D = [0.0625] * 4
    s = np.array([A + B + C + D], np.float32)
    idx, _ = oracle.route(s, np.zeros(16, np.float32), 4, 2, 4, 2, 1.0)
    assert idx[0].tolist() == [4, 5, 6, 7]


# ---------------------------------------------------------------- library special cases
def test_no_group_limit_no_bias_is_plain_topk():
    s = make_scores(1, 64, 32)
    idx, w = oracle.route(s, np.zeros(32, np.float32), 8, 8, 6, 2, 1.0)
    ref = np.argsort(-s.astype(np.float64), axis=1, kind="stable")[:, :6]
    assert (idx == ref).all()


def test_all_experts_selected_gives_affinity_share():
    s = make_scores(2, 16, 8)
    idx, w = oracle.route(s, np.zeros(8, np.float32), 4, 4, 8, 2, 2.5)
    full = np.zeros((16, 8))
    np.put_along_axis(full, idx.astype(np.int64), w, axis=1)
    s64 = s.astype(np.float64)
    np.testing.assert_allclose(full, 2.5 * s64 / s64.sum(1, keepdims=True), rtol=1e-14)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("E,G,M,k,r", [(16, 4, 2, 4, 2), (64, 8, 3, 6, 2), (256, 8, 4, 8, 2)])
def test_invariants_random(E, G, M, k, r):
    T = 128
    s = make_scores(3, T, E)
    b = (rng(4, E).uniform(-0.05, 0.05, E)).astype(np.float32)
    idx, w = oracle.route(s, b, G, M, k, r, 2.5)
    # gates sum to the scale
    assert np.abs(w.sum(1) - 2.5).max() <= k * np.spacing(2.5)
    # at most M groups per token, distinct experts
    for t in range(T):
        assert len(set((idx[t] // (E // G)).tolist())) <= M
        assert len(set(idx[t].tolist())) == k
    # slot order: biased score descending
    q = (s + b[None, :]).astype(np.float32)
    qs = np.take_along_axis(q, idx.astype(np.int64), 1)
    assert (np.diff(qs, axis=1) <= 0).all()
    # gates come from the raw affinity of the chosen expert
    sel = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), 1)
    assert (np.argsort(-w, axis=1, kind="stable") == np.argsort(-sel, axis=1, kind="stable")).all()


def test_uniform_bias_shift_changes_nothing():
    """b = c for every expert shifts every q and every group sum uniformly, so
    idx and the gates must be bit-identical to b = 0 (inputs on a 2^-12 grid
    keep s + c exact)."""
    E, G, M, k = 64, 8, 3, 6
    g = rng(5, 1)
    s = (g.integers(1, 4096, (200, E)) / 4096.0).astype(np.float32)
    idx0, w0 = oracle.route(s, np.zeros(E, np.float32), G, M, k, 2, 2.5)
    for c in (0.25, -0.125, 3.0):
        idx1, w1 = oracle.route(s, np.full(E, c, np.float32), G, M, k, 2, 2.5)
        assert (idx0 == idx1).all()
        assert (w0 == w1).all()


def test_bias_never_changes_gates_of_unchanged_sets():
    E, G, M, k = 64, 8, 3, 6
    s = make_scores(6, 500, E)
    b = rng(7, 2).uniform(-0.02, 0.02, E).astype(np.float32)
    idx0, w0 = oracle.route(s, np.zeros(E, np.float32), G, M, k, 2, 1.0)
    idx1, w1 = oracle.route(s, b, G, M, k, 2, 1.0)
    same = 0
    for t in range(500):
        if set(idx0[t].tolist()) == set(idx1[t].tolist()):
            same += 1
            d0 = dict(zip(idx0[t].tolist(), w0[t]))
            d1 = dict(zip(idx1[t].tolist(), w1[t]))
            for e in d0:
                assert abs(d0[e] - d1[e]) <= 1e-15
    assert 50 < same < 500   # the bias changed some selections but not all


def test_ties_resolved_to_lower_index_and_signed_zero():
    E, G, M, k = 16, 4, 2, 4
    s = make_scores(8, 300, E, kind="ties")
    idx, _ = oracle.route(s, np.zeros(E, np.float32), G, M, k, 2, 1.0)
    q = s.astype(np.float64)
    for t in range(300):
        _check_ties(q[t], idx[t], G, M, k)
    z = make_scores(9, 300, E, kind="zeros")
    assert np.signbit(z[z == 0]).any()
    idx_n, _ = oracle.route(z, np.zeros(E, np.float32), G, M, k, 2, 1.0)
    idx_p, _ = oracle.route(np.abs(z), np.zeros(E, np.float32), G, M, k, 2, 1.0)
    assert (idx_n == idx_p).all()   # -0.0 ranks exactly like +0.0
    for t in range(300):
        _check_ties(np.abs(z[t]).astype(np.float64), idx_n[t], G, M, k)


def _check_ties(qrow, idxrow, G, M, k):
    E = len(qrow)
    gsz = E // G
    gs = -np.sort(-qrow.reshape(G, gsz), axis=1)[:, :2].sum(1)
    # chosen groups: rank by (gs desc, g asc)
    order = sorted(range(G), key=lambda g: (-gs[g], g))[:M]
    allowed = [e for e in range(E) if e // gsz in order]
    exp = sorted(allowed, key=lambda e: (-qrow[e], e))[:k]
    assert idxrow.tolist() == exp


def test_diagnostics_worked_example():
    """Hand-derived margins of the worked example (k-th minus (k+1)-th biased score among
    the allowed experts; M-th minus (M+1)-th group score)."""
    g = _load("route_worked_example.json")
    s = np.array(g["scores"], np.float32)
    b = np.array(g["bias"], np.float32)
    gk, gm = oracle.route_diagnostics(s, b, g["G"], g["M"], g["k"], 2)
    assert gk.tolist() == g["r2_gaps"]["gap_k"]
    assert gm.tolist() == g["r2_gaps"]["gap_m"]
    gk1, gm1 = oracle.route_diagnostics(s, b, g["G"], g["M"], g["k"], 1)
    assert (gk1[0], gm1[0]) == (g["r1_token0_gaps"]["gap_k"], g["r1_token0_gaps"]["gap_m"])
    gk0, gm0 = oracle.route_diagnostics(s, np.zeros(8, np.float32), g["G"], g["M"], g["k"], 2)
    assert (gk0[0], gm0[0]) == (g["no_bias_token0_gaps"]["gap_k"], g["no_bias_token0_gaps"]["gap_m"])


@pytest.mark.parametrize("E,G,M,k,r", [(16, 4, 2, 4, 2), (12, 3, 2, 5, 3), (16, 8, 3, 4, 1)])
def test_diagnostics_brute_force(E, G, M, k, r):
    """The margins from enumeration: gap_m = the smallest group score among the best M-subset
    of groups minus the largest outside it; gap_k = the smallest biased score of the best
    k-subset of the allowed experts minus the largest allowed score outside it."""
    T = 30
    s, b = _dyadic_tie_free(E * 100 + G * 10 + M + 7, T, E, G, r)
    gk, gm = oracle.route_diagnostics(s, b, G, M, k, r)
    q = (s + b).astype(np.float64)
    gsz = E // G
    for t in range(T):
        row = list(q[t])
        gscore = [max(sum(c) for c in itertools.combinations(row[x * gsz:(x + 1) * gsz], r)) for x in range(G)]
        best_g = max(itertools.combinations(range(G), M), key=lambda gs: sum(gscore[x] for x in gs))
        rest_g = [x for x in range(G) if x not in best_g]
        exp_m = min(gscore[x] for x in best_g) - max(gscore[x] for x in rest_g) if rest_g else np.inf
        allowed = [e for e in range(E) if e // gsz in best_g]
        best = max(itertools.combinations(allowed, k), key=lambda es: sum(row[e] for e in es))
        rest = [e for e in allowed if e not in best]
        exp_k = min(row[e] for e in best) - max(row[e] for e in rest) if rest else np.inf
        assert gm[t] == pytest.approx(exp_m, rel=0, abs=1e-12)
        assert gk[t] == pytest.approx(exp_k, rel=0, abs=1e-12)


def test_diagnostics_gaps():
    E, G, M, k = 16, 4, 2, 4
    s = make_scores(10, 100, E, kind="ties")
    gk, gm = oracle.route_diagnostics(s, np.zeros(E, np.float32), G, M, k, 2)
    assert (gk >= 0).all() and (gm >= 0).all()
    assert (gk == 0).any() and (gm == 0).any()     # tie inputs produce exact ties
    s2 = make_scores(11, 100, E)
    gk2, gm2 = oracle.route_diagnostics(s2, np.zeros(E, np.float32), G, M, k, 2)
    assert (gk2 > 0).all() and (gm2 > 0).all()
    gk3, gm3 = oracle.route_diagnostics(s2, np.zeros(E, np.float32), G, G, E, 2)
    assert np.isinf(gk3).all() and np.isinf(gm3).all()


def test_affinity_is_sigmoid_of_logits():
    x = rng(12, 1).standard_normal((20, 32))
    wr = rng(12, 2).standard_normal((8, 32)) * 0.1
    o = rng(12, 3).standard_normal(8)
    s = oracle.affinity(x, wr, o)
    from scipy.special import expit
    ref = expit(x @ wr.T + o).astype(np.float32)
    assert s.dtype == np.float32
    assert (s == ref).all()
