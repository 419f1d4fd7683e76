"""Oracle: per-expert load count and the expert-sorted permutation (dispatch).

TEST INFRASTRUCTURE (see the package docstring).

Dispatch sends every token to the experts it selected (DeepSeek-V3 Technical
Report：中英对照解读, §2.2: expert parallelism needs token dispatch and combine).
On one GPU that is a permutation of the (token, slot) pairs into per-expert
contiguous segments.  The load of an expert is the number of pairs routed to it
over the whole batch (qwbw.cn essay, load-balancing section: loads are counted
over the whole batch after each step).

Reading: the permutation is the stable sort of the flat pair ids f = t*k + j by
expert, so each segment lists its pairs in increasing f; inv[t, j] is the row
of pair (t, j) in the permuted order.
"""
from __future__ import annotations

import numpy as np


def dispatch(idx: np.ndarray, n_experts: int):
    """Returns counts [E], offsets [E+1], perm [T*k] (flat pair ids), inv [T, k]."""
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(flat, kind="stable")
    inv = np.empty(T * k, dtype=np.int64)
    inv[perm] = np.arange(T * k)
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
            inv.reshape(T, k).astype(np.int32))


def permute_rows(x: np.ndarray, perm: np.ndarray, top_k: int) -> np.ndarray:
    """x_perm[p] = x[perm[p] // k]: each pair's row is its token's activation."""
    return np.asarray(x)[np.asarray(perm, np.int64) // top_k]
