"""Pins of the oracle's dispatch, combine and bias update."""
import json
import os

import numpy as np

import oracle
from workloads.inputs import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _idx(seed, T, E, k):
    g = rng(seed, 5)
    return np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)


# ---------------------------------------------------------------- dispatch
def test_dispatch_segments_by_enumeration():
    T, E, k = 97, 13, 3
    idx = _idx(1, T, E, k)
    counts, offsets, perm, inv = oracle.dispatch(idx, E)
    assert offsets[0] == 0 and offsets[-1] == T * k
    for e in range(E):
        members = [t * k + j for t in range(T) for j in range(k) if idx[t, j] == e]   # ascending f
        assert counts[e] == len(members)
        assert perm[offsets[e]:offsets[e + 1]].tolist() == members
    for t in range(T):
        for j in range(k):
            assert perm[inv[t, j]] == t * k + j
    assert sorted(perm.tolist()) == list(range(T * k))


def test_dispatch_empty_experts_and_single_expert():
    idx = np.zeros((5, 1), np.int32) + 2
    counts, offsets, perm, inv = oracle.dispatch(idx, 4)
    assert counts.tolist() == [0, 0, 5, 0]
    assert offsets.tolist() == [0, 0, 0, 5, 5]
    assert perm.tolist() == [0, 1, 2, 3, 4]
    assert inv[:, 0].tolist() == [0, 1, 2, 3, 4]


def test_permute_rows():
    T, E, k, H = 20, 6, 2, 5
    idx = _idx(2, T, E, k)
    x = np.arange(T * H, dtype=np.float32).reshape(T, H)
    _, offsets, perm, inv = oracle.dispatch(idx, E)
    xp = oracle.permute_rows(x, perm, k)
    for t in range(T):
        for j in range(k):
            assert (xp[inv[t, j]] == x[t]).all()
            e = idx[t, j]
            assert offsets[e] <= inv[t, j] < offsets[e + 1]


# ---------------------------------------------------------------- combine
def test_combine_single_slot_is_gather():
    T, E, k, H = 30, 5, 1, 7
    idx = _idx(3, T, E, k)
    _, _, perm, inv = oracle.dispatch(idx, E)
    yp = rng(4, 1).standard_normal((T * k, H))
    y = oracle.combine(yp, None, inv, np.ones((T, 1)))
    assert (y == yp[inv[:, 0]]).all()


def test_combine_matches_hand_sum():
    inv = np.array([[1, 2], [0, 3]])
    w = np.array([[0.5, 0.25], [2.0, -1.0]])
    yp = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    ysh = np.array([[10.0, 20.0], [30.0, 40.0]])
    y = oracle.combine(yp, ysh, inv, w)
    # token 0: 10 + 0.5*[3,4] + 0.25*[5,6] = [12.75, 23.5]; token 1: 30 + 2*[1,2] - [7,8] = [25, 36]
    assert y.tolist() == [[12.75, 23.5], [25.0, 36.0]]


# ---------------------------------------------------------------- bias update
def test_bias_update_hand_fixture():
    with open(os.path.join(GOLDEN, "bias_update_example.json")) as f:
        g = json.load(f)
    b = np.array(g["bias"], np.float32)
    c = np.array(g["counts"], np.int32)
    out0 = oracle.update_bias(b, c, g["T"], g["k"], g["gamma"], 0)
    out1 = oracle.update_bias(b, c, g["T"], g["k"], g["gamma"], 1)
    assert out0.tolist() == g["mode0_expected"]
    assert out1.tolist() == g["mode1_expected"]
    assert out0.dtype == np.float32


def test_bias_moves_exactly_gamma_each_step():
    E = 256
    g = rng(9, 1)
    b = g.uniform(-0.01, 0.01, E).astype(np.float32)
    c = g.integers(0, 1100, E).astype(np.int32)
    new = oracle.update_bias(b, c, 16384, 8, 1e-3)
    gam = np.float32(1e-3)
    over = c.astype(np.int64) * E > 16384 * 8
    assert (new[over] == (b[over] - gam)).all()
    assert (new[~over] == (b[~over] + gam)).all()
    assert (new != b).all()
    # zero gamma is a fixed point
    assert (oracle.update_bias(b, c, 16384, 8, 0.0) == b).all()


def test_feedback_flip_step_closed_form():
    """Three experts, one token preferring A (s = .75, .5, .25), k = 1, one group,
    gamma = 2^-6.  While A is picked its bias falls and the others rise by gamma
    per step, so A stays picked while 0.75 - n*g >= 0.5 + n*g (a tie keeps the
    lower index A): steps 0..8; the first step that picks B is n = 9."""
    s = np.array([[0.75, 0.5, 0.25]], np.float32)
    b = np.zeros(3, np.float32)
    gamma = 2.0 ** -6
    picks = []
    for n in range(12):
        idx, _ = oracle.route(s, b, 1, 1, 1, 1, 1.0)
        counts, _, _, _ = oracle.dispatch(idx, 3)
        picks.append(int(idx[0, 0]))
        b = oracle.update_bias(b, counts, 1, 1, gamma)
    assert picks[:9] == [0] * 9
    assert picks[9] == 1


def test_balancing_reduces_skew():
    """Many tokens crowding one expert (the product page's routing widget shows
    tokens rushing to expert A under raw preference); repeated bias updates on
    the same batch spread the load: max/mean falls."""
    T, E, k = 512, 16, 2
    g = rng(10, 1)
    logits = g.standard_normal((T, E)) * 0.5
    logits[:, 0] += 2.0
    s = (1.0 / (1.0 + np.exp(-logits))).astype(np.float32)
    b = np.zeros(E, np.float32)
    ratios = []
    for _ in range(400):
        idx, _ = oracle.route(s, b, 4, 4, k, 2, 1.0)
        counts, _, _, _ = oracle.dispatch(idx, E)
        ratios.append(counts.max() / (T * k / E))
        b = oracle.update_bias(b, counts, T, k, 1e-3)
    assert ratios[0] > 3.0
    assert max(ratios[-20:]) < 1.5
