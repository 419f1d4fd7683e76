"""Oracle: token-to-expert affinity and biased, group-limited top-k routing.

TEST INFRASTRUCTURE (see the package docstring).

What the pages fix:
* each routed expert i carries a bias b_i that takes part only in choosing the
  top-K experts; the gating value that multiplies an expert's output comes from
  the original score, never from the bias (DeepSeek-V3 Technical Report reading
  notes, Method §1 "Auxiliary-loss-free 负载均衡"; DeepSeek-V3 Technical
  Report：中英对照解读, §3; DeepSeek V3 product page, the "公式解密" box, which
  writes the ranking score as affinity plus bias);
* a token is sent to at most M nodes (reading notes, Method §1; qwbw.cn essay,
  section on the training infrastructure).  On one GPU the nodes become M of G
  contiguous expert groups.

Readings where the pages are silent (each a parameter, never hidden):
* affinity s = sigmoid(x W_r^T + o), rounded once to fp32;
* biased score q = fl32(s + b);
* group score = fl32 sum of the group's top-r values of q, added from the
  largest down (r = group_topr);
* two stages: the M groups with the largest group score, then the k largest q
  among the experts of those groups; ties go to the lower group / expert index
  and -0.0 counts as +0.0; slots are ordered by q descending, then index;
* gates w_j = scale * s_j / sum_j' s_j' over the selected experts (fp64 here).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
F32 = np.float32


def affinity(x: np.ndarray, w_router: np.ndarray, logit_offset=None) -> np.ndarray:
    """s[t, e] = sigmoid(<x_t, w_e> + o_e) computed in fp64, then rounded to fp32.

    x and w_router are already-decoded real values (any float dtype).
    """
    logits = np.asarray(x, F64) @ np.asarray(w_router, F64).T
    if logit_offset is not None:
        logits = logits + np.asarray(logit_offset, F64)[None, :]
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-logits))
    return s.astype(F32)


def _biased(s32: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """q = fl32(s + b): one fp32 add per element."""
    return (np.asarray(s32, F32) + np.asarray(bias, F32)[None, :]).astype(F32)


def _group_scores(q: np.ndarray, n_groups: int, topr: int) -> np.ndarray:
    """Sum (fp32, largest first) of the top-`topr` biased scores of each group."""
    T, E = q.shape
    qg = q.reshape(T, n_groups, E // n_groups)
    desc = -np.sort(-qg, axis=2)          # each group's scores, largest first
    gs = desc[:, :, 0].copy()
    for i in range(1, topr):
        gs = (gs + desc[:, :, i]).astype(F32)
    return gs


def route(s32: np.ndarray, bias: np.ndarray, n_groups: int, groups_per_token: int,
          top_k: int, group_topr: int, route_scale: float):
    """Biased, group-limited top-k.  Returns (idx int32 [T,k], w float64 [T,k]).

    idx[t, j] is the j-th selected expert (q descending, index ascending);
    w[t, j] = scale * s[t, idx] / sum over the selected experts of s.
    """
    s32 = np.asarray(s32, F32)
    T, E = s32.shape
    gsz = E // n_groups
    q = _biased(s32, bias)
    gs = _group_scores(q, n_groups, group_topr)
    # stable sort of the negated scores: larger first, ties keep the lower index first
    chosen = np.argsort(-gs, axis=1, kind="stable")[:, :groups_per_token]
    group_of = np.arange(E) // gsz
    allowed = (group_of[None, :, None] == chosen[:, None, :]).any(axis=2)
    qm = np.where(allowed, q.astype(F64), -np.inf)
    idx = np.argsort(-qm, axis=1, kind="stable")[:, :top_k]
    sel = np.take_along_axis(s32.astype(F64), idx, axis=1)
    w = route_scale * sel / sel.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w


def route_diagnostics(s32: np.ndarray, bias: np.ndarray, n_groups: int, groups_per_token: int,
                      top_k: int, group_topr: int):
    """Per-token margins of the two selections (fp64 differences of fp32 values).

    gap_k[t] = q_(k) - q_(k+1) among the allowed experts (inf if none follows);
    gap_m[t] = gs_(M) - gs_(M+1) over groups (inf if M == G).
    A GPU index that differs from the oracle's at token t is a near-tie, not an
    error, when either gap is below the stated threshold.
    """
    s32 = np.asarray(s32, F32)
    T, E = s32.shape
    gsz = E // n_groups
    q = _biased(s32, bias)
    gs = _group_scores(q, n_groups, group_topr).astype(F64)
    gsd = -np.sort(-gs, axis=1)
    gap_m = (gsd[:, groups_per_token - 1] - gsd[:, groups_per_token]
             if groups_per_token < n_groups else np.full(T, np.inf))
    chosen = np.argsort(-gs, axis=1, kind="stable")[:, :groups_per_token]
    group_of = np.arange(E) // gsz
    allowed = (group_of[None, :, None] == chosen[:, None, :]).any(axis=2)
    qd = -np.sort(-np.where(allowed, q.astype(F64), -np.inf), axis=1)
    n_allowed = groups_per_token * gsz
    gap_k = (qd[:, top_k - 1] - qd[:, top_k] if top_k < n_allowed else np.full(T, np.inf))
    return gap_k, gap_m
