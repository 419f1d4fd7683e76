"""Oracle: combine the routed expert outputs with their gates.

TEST INFRASTRUCTURE (see the package docstring).

After the experts run, each token's results are gathered back (DeepSeek-V3
Technical Report：中英对照解读, §2.2: dispatch and combine) and weighted by the
gating values, which come from the raw affinities (reading notes, Method §1).
Reading: no residual is added; the layer returns shared + routed, summed in
fp64 with the slots in ascending j.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def combine(y_perm: np.ndarray, y_shared, inv: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[t] = y_shared[t] + sum_j w[t, j] * y_perm[inv[t, j]]  (fp64)."""
    inv = np.asarray(inv, np.int64)
    w = np.asarray(w, F64)
    T, k = inv.shape
    y = np.zeros((T, y_perm.shape[1]), F64) if y_shared is None else np.array(y_shared, F64)
    for j in range(k):
        y += w[:, j:j + 1] * np.asarray(y_perm, F64)[inv[:, j]]
    return y
