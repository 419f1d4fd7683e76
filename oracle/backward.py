"""Oracle: gradients of one MoE layer pass, and the sequence-wise balance loss.

TEST INFRASTRUCTURE (see the package docstring).

The forward being differentiated is the one the rest of the oracle states:
    y_t = sum_s FFN_s(x_t) + sum_j w_tj FFN_{e_tj}(x_t),
    w_tj = scale * s_{t,e_tj} / sum_j' s_{t,e_tj'},   s = sigmoid(x W_r^T + o),
with FFN(v) = W_d (silu(W_g v) * W_u v) (DeepSeek-V3 Technical Report：中英对照解读,
§2 and §3).  The expert choice e_tj (biased, group-limited top-k) is piecewise
constant, so it carries no gradient; the bias takes part only in that choice,
so it gets none either (reading notes, Method §1: the bias is used for routing
only, the gate comes from the original score).

The pages keep "a small sequence-wise balance loss" with a very small weight
alpha against extreme imbalance inside one sequence (reading notes, Method §1
and the bilingual notes' list of auxiliary terms), but print no formula.
Reading used here (every symbol a parameter):
    the batch is T / L sequences of L consecutive tokens; for sequence b
        f_e = E / (k L) * #{t in b : e is one of t's selected experts}
        P_e = (1 / L) * sum_{t in b} s_te / sum_e' s_te'
        L_b = alpha * sum_e f_e P_e
    and the loss is the mean of L_b over the sequences.  f counts the experts
    the layer actually selects (biased, group-limited), so it is a constant
    for the gradient, which flows through P into the affinities.
All arithmetic is fp64; inputs are already-decoded real values.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def gate_backward(s_sel: np.ndarray, dw: np.ndarray, scale: float) -> np.ndarray:
    """d loss / d s at the selected experts, given d loss / d w.

    w_j = c s_j / S with S = sum_j s_j, so dw_j/ds_i = c (delta_ij / S - s_j / S^2) and
    ds_i = (c / S) (dw_i - sum_j dw_j s_j / S).   s_sel, dw: [T, k]."""
    s_sel = np.asarray(s_sel, F64)
    dw = np.asarray(dw, F64)
    S = s_sel.sum(axis=1, keepdims=True)
    return (scale / S) * (dw - (dw * s_sel).sum(axis=1, keepdims=True) / S)


def seq_balance_loss(s: np.ndarray, idx: np.ndarray, k: int, seq_len: int, alpha: float):
    """(loss, d loss / d s [T, E]) of the sequence-wise balance loss read above."""
    s = np.asarray(s, F64)
    T, E = s.shape
    assert T % seq_len == 0, "whole sequences"
    B = T // seq_len
    hit = np.zeros((T, E), F64)
    np.put_along_axis(hit, np.asarray(idx, np.int64), 1.0, axis=1)
    row_sum = s.sum(axis=1, keepdims=True)
    sn = s / row_sum                                        # s'_te
    loss = 0.0
    g = np.zeros((T, E), F64)                               # d loss / d s'
    for b in range(B):
        rows = slice(b * seq_len, (b + 1) * seq_len)
        f = E / (k * seq_len) * hit[rows].sum(axis=0)       # [E]
        P = sn[rows].mean(axis=0)                           # [E]
        loss += alpha * float((f * P).sum()) / B
        g[rows] = alpha / B * f[None, :] / seq_len
    # s' = s / sum(s): ds_i = g_i / S - sum_e g_e s_e / S^2
    ds = g / row_sum - (g * s).sum(axis=1, keepdims=True) / row_sum ** 2
    return loss, ds


def swiglu_backward(X: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray, dY: np.ndarray):
    """Gradients of Y = W_d (silu(W_g X) * W_u X) for one expert on rows X [n, H].

    Returns (dX [n, H], dW_gate_up [2I, H], dW_down [H, I], h [n, I])."""
    X = np.asarray(X, F64)
    Wgu = np.asarray(w_gate_up, F64)
    Wd = np.asarray(w_down, F64)
    dY = np.asarray(dY, F64)
    I = Wgu.shape[0] // 2
    a = X @ Wgu[:I].T
    u = X @ Wgu[I:].T
    sg = _sigmoid(a)
    silu = a * sg
    h = silu * u
    dh = dY @ Wd                          # [n, I]
    dWd = dY.T @ h                        # [H, I]
    du = dh * silu
    da = dh * u * (sg + a * sg * (1.0 - sg))
    dWgu = np.concatenate([da.T @ X, du.T @ X], axis=0)
    dX = da @ Wgu[:I] + du @ Wgu[I:]
    return dX, dWgu, dWd, h


def backward_from_routing(x, w_router, logit_offset, w_gate_up, w_down, ws_gate_up, ws_down,
                          idx, dy, scale: float, alpha: float = 0.0, seq_len: int = 0):
    """All gradients of sum(dy * y) + L_bal for fixed expert choices idx [T, k].

    x [T, H], w_router [E, H], logit_offset [E] or None, w_gate_up [E, 2I, H],
    w_down [E, H, I], ws_* [S, ...] (S may be 0), dy [T, H]; alpha = 0 drops the
    balance loss.  Returns a dict of fp64 arrays: the layer output y, the
    intermediates (s, w, y_perm rows per (t, j), dw, ds, dlogit) and the gradients
    dx, dw_router, dw_gate_up, dw_down, dws_gate_up, dws_down, plus loss_bal."""
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    idx = np.asarray(idx, np.int64)
    T, H = x.shape
    E = w_router.shape[0]
    k = idx.shape[1]
    logits = x @ np.asarray(w_router, F64).T
    if logit_offset is not None:
        logits = logits + np.asarray(logit_offset, F64)[None, :]
    s = _sigmoid(logits)
    s_sel = np.take_along_axis(s, idx, axis=1)
    w = scale * s_sel / s_sel.sum(axis=1, keepdims=True)

    y = np.zeros((T, H), F64)
    dx = np.zeros((T, H), F64)
    dw = np.zeros((T, k), F64)
    y_slot = np.zeros((T, k, H), F64)
    dWgu = np.zeros(np.shape(w_gate_up), F64)
    dWd = np.zeros(np.shape(w_down), F64)
    for e in range(E):
        t_of, j_of = np.nonzero(idx == e)
        if len(t_of) == 0:
            continue
        X = x[t_of]
        # expert output (ungated) on its rows
        Wgu = np.asarray(w_gate_up[e], F64)
        I = Wgu.shape[0] // 2
        a = X @ Wgu[:I].T
        hh = a * _sigmoid(a) * (X @ Wgu[I:].T)
        Ye = hh @ np.asarray(w_down[e], F64).T
        y_slot[t_of, j_of] = Ye
        gate = w[t_of, j_of][:, None]
        y[t_of] += gate * Ye
        dw[t_of, j_of] = (dy[t_of] * Ye).sum(axis=1)
        dXe, dWgu[e], dWd[e], _ = swiglu_backward(X, w_gate_up[e], w_down[e], gate * dy[t_of])
        np.add.at(dx, t_of, dXe)
    S = 0 if ws_gate_up is None else len(ws_gate_up)
    dWsgu = np.zeros(np.shape(ws_gate_up), F64) if S else None
    dWsd = np.zeros(np.shape(ws_down), F64) if S else None
    for sh in range(S):
        Wgu = np.asarray(ws_gate_up[sh], F64)
        I = Wgu.shape[0] // 2
        a = x @ Wgu[:I].T
        y += (a * _sigmoid(a) * (x @ Wgu[I:].T)) @ np.asarray(ws_down[sh], F64).T
        dXs, dWsgu[sh], dWsd[sh], _ = swiglu_backward(x, ws_gate_up[sh], ws_down[sh], dy)
        dx += dXs

    ds = np.zeros((T, E), F64)
    np.put_along_axis(ds, idx, gate_backward(s_sel, dw, scale), axis=1)
    loss_bal = 0.0
    if alpha:
        loss_bal, ds_bal = seq_balance_loss(s, idx, k, seq_len or T, alpha)
        ds += ds_bal
    dlogit = ds * s * (1.0 - s)
    dWr = dlogit.T @ x
    dx += dlogit @ np.asarray(w_router, F64)
    return dict(y=y, s=s, w=w, y_slot=y_slot, dw=dw, ds=ds, dlogit=dlogit, loss_bal=loss_bal,
                dx=dx, dw_router=dWr, dw_gate_up=dWgu, dw_down=dWd, dws_gate_up=dWsgu, dws_down=dWsd)
