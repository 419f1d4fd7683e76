"""Oracle: the SwiGLU experts (routed, per segment, and shared, over all tokens).

TEST INFRASTRUCTURE (see the package docstring).

The layer has shared experts that every token passes through plus routed
experts chosen by top-k (DeepSeek-V3 Technical Report：中英对照解读, §2
Architecture, "Shared experts and routed experts").  The pages never name the
expert's form; the reading here is a SwiGLU FFN without biases:
    FFN(x) = W_d (silu(W_g x) * (W_u x)),   silu(a) = a / (1 + exp(-a)).
Weights are [out, in]; w_gate_up stacks the gate rows [0, I) above the up rows
[I, 2I).  All arithmetic is fp64 on already-decoded values.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def swiglu(X: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One expert on rows X [n, H]: returns [n, H] in fp64."""
    X = np.asarray(X, F64)
    w_gate_up = np.asarray(w_gate_up, F64)
    I = w_gate_up.shape[0] // 2
    a = X @ w_gate_up[:I].T
    u = X @ w_gate_up[I:].T
    with np.errstate(over="ignore"):
        h = a / (1.0 + np.exp(-a)) * u
    return h @ np.asarray(w_down, F64).T


def routed_ffn(x_perm: np.ndarray, offsets: np.ndarray, w_gate_up, w_down) -> np.ndarray:
    """y_perm[p] = FFN_e(x_perm[p]) for the expert e whose segment holds row p."""
    n, H = x_perm.shape
    y = np.zeros((n, H), F64)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi] = swiglu(x_perm[lo:hi], w_gate_up[e], w_down[e])
    return y


def shared_ffn(x: np.ndarray, ws_gate_up, ws_down) -> np.ndarray:
    """Sum over the shared experts of FFN_s(x); zeros when there are none."""
    y = np.zeros((x.shape[0], x.shape[1]), F64)
    for s in range(len(ws_gate_up)):
        y += swiglu(x, ws_gate_up[s], ws_down[s])
    return y
