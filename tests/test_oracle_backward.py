"""Pins of the backward oracle (CPU only).

* Every gradient against central finite differences of an independent fp64
  forward written here from the layer's definition (oracle.swiglu for the
  experts, the gate and the balance loss restated), with the expert choice held
  fixed: the function is then smooth, so the differences converge.
* The balance-loss value on a hand-computed example and on the closed form of
  uniform affinities (loss = alpha); the gate gradient is zero when k = 1 (the
  gate is the constant `scale`).
"""
import numpy as np
import pytest

import oracle
from oracle.backward import backward_from_routing, gate_backward, seq_balance_loss

F64 = np.float64


def _case(seed=0, T=8, H=6, E=8, k=2, S=1, I=3):
    r = np.random.default_rng(seed)
    p = dict(x=r.normal(size=(T, H)), wr=r.normal(0, 0.5, (E, H)), off=r.normal(size=E),
             wgu=r.normal(0, 0.5, (E, 2 * I, H)), wd=r.normal(0, 0.5, (E, H, I)),
             wsgu=r.normal(0, 0.5, (S, 2 * I, H)), wsd=r.normal(0, 0.5, (S, H, I)))
    dy = r.normal(size=(T, H))
    s = 1.0 / (1.0 + np.exp(-(p["x"] @ p["wr"].T + p["off"])))
    idx = np.argsort(-s, axis=1, kind="stable")[:, :k]        # any fixed choice will do
    return p, dy, idx


def _total(p, dy, idx, scale, alpha, L):
    """sum(dy * y) + balance loss, from the definitions (no gradient code)."""
    x = p["x"]
    T, k = idx.shape
    E = p["wr"].shape[0]
    s = 1.0 / (1.0 + np.exp(-(x @ p["wr"].T + p["off"])))
    sel = np.take_along_axis(s, idx, axis=1)
    w = scale * sel / sel.sum(axis=1, keepdims=True)
    y = np.zeros_like(x)
    for sh in range(len(p["wsgu"])):
        y += oracle.swiglu(x, p["wsgu"][sh], p["wsd"][sh])
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            y[t] += w[t, j] * oracle.swiglu(x[t:t + 1], p["wgu"][e], p["wd"][e])[0]
    total = float((dy * y).sum())
    if alpha:
        sn = s / s.sum(axis=1, keepdims=True)
        for b in range(T // L):
            rows = range(b * L, (b + 1) * L)
            cnt = np.zeros(E)
            for t in rows:
                for j in range(k):
                    cnt[idx[t, j]] += 1
            f = E / (k * L) * cnt
            P = sn[list(rows)].mean(axis=0)
            total += alpha * float((f * P).sum()) / (T // L)
    return total


def _grads(p, dy, idx, scale, alpha, L):
    return backward_from_routing(p["x"], p["wr"], p["off"], p["wgu"], p["wd"], p["wsgu"], p["wsd"], idx, dy,
                                 scale, alpha, L)


@pytest.mark.parametrize("alpha,L", [(0.0, 8), (0.3, 4), (0.3, 8)])
def test_gradients_match_finite_differences(alpha, L):
    p, dy, idx = _case()
    scale = 2.5
    g = _grads(p, dy, idx, scale, alpha, L)
    names = dict(x="dx", wr="dw_router", wgu="dw_gate_up", wd="dw_down", wsgu="dws_gate_up", wsd="dws_down")
    eps = 1e-5
    for key, gname in names.items():
        a = p[key]
        fd = np.zeros_like(a)
        for i in np.ndindex(a.shape):
            old = a[i]
            a[i] = old + eps
            up = _total(p, dy, idx, scale, alpha, L)
            a[i] = old - eps
            dn = _total(p, dy, idx, scale, alpha, L)
            a[i] = old
            fd[i] = (up - dn) / (2 * eps)
        an = g[gname]
        err = np.abs(fd - an).max() / max(np.abs(an).max(), 1e-12)
        assert err < 1e-6, f"{gname}: relative error {err:.2e}"


def test_forward_value_and_loss_agree_with_definition():
    p, dy, idx = _case(seed=3)
    g = _grads(p, dy, idx, 1.7, 0.2, 4)
    total = _total(p, dy, idx, 1.7, 0.2, 4)
    assert abs(float((dy * g["y"]).sum()) + g["loss_bal"] - total) < 1e-10 * max(1.0, abs(total))


def test_balance_loss_hand_example():
    # one sequence of two tokens, four experts, k = 1, both tokens on expert 0:
    # f = 4 / (1 * 2) * [2, 0, 0, 0] = [4, 0, 0, 0]; the rows already sum to 1, so
    # P_0 = (0.5 + 0.2) / 2 = 0.35 and the loss is alpha * 4 * 0.35 = 1.4 alpha
    s = np.array([[0.5, 0.25, 0.125, 0.125], [0.2, 0.2, 0.3, 0.3]])
    idx = np.array([[0], [0]])
    loss, _ = seq_balance_loss(s, idx, 1, 2, 0.01)
    assert abs(loss - 0.014) < 1e-15


def test_balance_loss_uniform_closed_form():
    # equal affinities: P_e = 1/E for every expert and sum_e f_e = E, so loss = alpha
    r = np.random.default_rng(1)
    T, E, k, L = 12, 16, 3, 4
    s = np.full((T, E), 0.37)
    idx = np.stack([r.choice(E, k, replace=False) for _ in range(T)])
    loss, ds = seq_balance_loss(s, idx, k, L, 0.05)
    assert abs(loss - 0.05) < 1e-15
    # moving all affinities of a token by the same factor leaves s' unchanged
    assert np.abs((ds * s).sum(axis=1)).max() < 1e-15


def test_gate_gradient_vanishes_for_single_expert():
    s = np.random.default_rng(2).uniform(0.1, 0.9, (5, 1))
    assert np.abs(gate_backward(s, np.ones((5, 1)), 2.5)).max() == 0.0
