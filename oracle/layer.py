"""Oracle: one MoE layer forward, step by step, plus a per-token sampled variant.

TEST INFRASTRUCTURE (see the package docstring).

Order of the steps: affinity -> biased group-limited top-k -> load count and
dispatch -> routed and shared SwiGLU experts -> gated combine -> bias update
for the next batch (DeepSeek-V3 Technical Report：中英对照解读, §2 and §3;
reading notes, Method §1).  With wgt == "fp8_e4m3" the expert GEMMs follow the
fine-grained FP8 recipe of oracle.fp8 (qwbw.cn essay, FP8 part of the
infrastructure section): x and h per 1x128 tile, weights per 128x128 block,
while routing stays in higher precision (the same section keeps MoE gating in
BF16/FP32).

`cfg` is any object with the attributes T H E G M k S I group_topr route_scale
act wgt gamma bias_eq_mode.  Stored tensors are either float32 values or bf16
bit patterns (uint16), decoded here.
"""
from __future__ import annotations

import numpy as np

from .balance import update_bias
from .combine import combine
from .dispatch import dispatch, permute_rows
from .ffn import swiglu
from .fp8 import fp8_matmul, quantize_blocks_128x128, quantize_rows_1x128
from .route import affinity, route

F64 = np.float64
F32 = np.float32


def decode_act(a: np.ndarray) -> np.ndarray:
    """float32 values pass through; uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(F32)
    return a.astype(F32, copy=False)


def _silu_mul(a: np.ndarray, u: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a)) * u


class _Fp8Expert:
    """One expert's weights quantised per 128x128 block (offline weight prep)."""

    def __init__(self, w_gate_up, w_down):
        self.qgu, self.sgu = quantize_blocks_128x128(decode_act(w_gate_up))
        self.qd, self.sd = quantize_blocks_128x128(decode_act(w_down))
        self.I = self.qgu.shape[0] // 2

    def hidden(self, qx, sx):
        """SwiGLU intermediate h (fp64) of rows given as 1x128 E4M3 tiles."""
        ab = fp8_matmul(qx, sx, self.qgu, self.sgu)
        return _silu_mul(ab[:, :self.I], ab[:, self.I:])

    def down(self, qh, sh):
        """Down projection of an E4M3-quantised h (fp64)."""
        return fp8_matmul(qh, sh, self.qd, self.sd)

    def __call__(self, qx, sx):
        qh, sh = quantize_rows_1x128(self.hidden(qx, sx).astype(F32))
        return self.down(qh, sh)


def _expert_fn(cfg, w_gate_up, w_down):
    if cfg.wgt == "fp8_e4m3":
        ex = _Fp8Expert(w_gate_up, w_down)
        return lambda rows_q: ex(*rows_q)
    wgu = decode_act(w_gate_up)
    wd = decode_act(w_down)
    return lambda rows: swiglu(rows, wgu, wd)


def _rows_view(cfg, x32):
    """What an expert consumes: fp64 rows, or (codes, scales) of 1x128 tiles for fp8."""
    if cfg.wgt == "fp8_e4m3":
        return quantize_rows_1x128(x32)
    return x32.astype(F64)


def _take(view, rows):
    if isinstance(view, tuple):
        return (view[0][rows], view[1][rows])
    return view[rows]


def layer_forward(cfg, x, weights, bias, scores_in=None):
    """The whole layer over all T tokens.  Returns a dict of every intermediate.

    scores_in: optional fp32 affinities to route on instead of computing them
    (used when the routing is teacher-forced with another implementation's s).
    """
    x32 = decode_act(x)
    if scores_in is None:
        s32 = affinity(x32, decode_act(weights.w_router), weights.logit_offset)
    else:
        s32 = np.asarray(scores_in, F32)
    idx, w = route(s32, bias, cfg.G, cfg.M, cfg.k, cfg.group_topr, cfg.route_scale)
    return forward_from_routing(cfg, x, weights, bias, s32, idx, w)


def forward_from_routing(cfg, x, weights, bias, s32, idx, w):
    x32 = decode_act(x)
    counts, offsets, perm, inv = dispatch(idx, cfg.E)
    view = _rows_view(cfg, x32)
    xp = _take(view, np.asarray(perm, np.int64) // cfg.k)
    y_perm = np.zeros((cfg.T * cfg.k, cfg.H), F64)
    for e in range(cfg.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            f = _expert_fn(cfg, weights.w_gate_up[e], weights.w_down[e])
            y_perm[lo:hi] = f(_take(xp, slice(lo, hi)))
    y_sh = np.zeros((cfg.T, cfg.H), F64)
    for s in range(cfg.S):
        y_sh += _expert_fn(cfg, weights.ws_gate_up[s], weights.ws_down[s])(view)
    y = combine(y_perm, y_sh, inv, w)
    new_bias = update_bias(bias, counts, cfg.T, cfg.k, cfg.gamma, getattr(cfg, "bias_eq_mode", 0))
    return dict(s32=s32, idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv,
                x_perm=permute_rows(x, perm, cfg.k), y_perm=y_perm, y_shared=y_sh, y=y,
                bias_next=new_bias)


def sampled_forward(cfg, x_rows, idx_rows, w_rows, weights, experts_cache=None):
    """Layer output for a subset of tokens, given their routing (tokens are
    independent once routed).  x_rows [n, H] stored values; idx_rows, w_rows [n, k].
    Returns y_rows [n, H] fp64 (shared + gated routed outputs).
    experts_cache: optional dict that keeps each expert's prepared form (keys e for
    routed experts, ("shared", s) for shared ones) between calls."""
    x32 = decode_act(x_rows)
    view = _rows_view(cfg, x32)
    n = x32.shape[0]
    y = np.zeros((n, cfg.H), F64)
    cache = {} if experts_cache is None else experts_cache

    def expert(key, w_gate_up, w_down):
        if key not in cache:
            cache[key] = _expert_fn(cfg, w_gate_up, w_down)
        return cache[key]

    for s in range(cfg.S):
        y += expert(("shared", s), weights.ws_gate_up[s], weights.ws_down[s])(view)
    idx_rows = np.asarray(idx_rows)
    w_rows = np.asarray(w_rows, F64)
    for e in np.unique(idx_rows):
        r, j = np.nonzero(idx_rows == e)
        f = expert(int(e), weights.w_gate_up[e], weights.w_down[e])
        ye = f(_take(view, r))
        y[r] += w_rows[r, j][:, None] * ye
    return y
