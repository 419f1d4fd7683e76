"""Seeded synthetic inputs for the MoE-layer workloads.

Every tensor has its own child stream of numpy's PCG64, keyed by
(seed, tensor tag, index...), so tensors can be generated in parallel and
independently of one another (x of step 7 does not depend on how many experts
were drawn).  Values:

* activations x ~ N(0, 1); every weight ~ N(0, sigma) with sigma the std-dev;
* router logit offsets: N(0, 1) per expert, or a Zipf(s) preference
  o_e = ln(E * p_rank(e)) with p_r proportional to r^-s over ranks 1..E and a
  seeded random rank per expert (so hot experts are spread over groups);
* initial bias: zero or U(-r, r).

bf16 tensors are returned as their uint16 bit patterns (numpy has no bf16),
rounded once from the float32 draw with round-to-nearest-even; fp32 tensors are
the float32 draw itself.  This module is the only code shared by the oracle's
callers and the GPU path's callers, and it holds none of the layer's arithmetic.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import MoeConfig

TAG_X, TAG_WR, TAG_OFF, TAG_PERM, TAG_BIAS, TAG_WGU, TAG_WD, TAG_SGU, TAG_SD, TAG_SCORES = range(1, 11)
X_CHUNK_ROWS = 1024


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *tags])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def _normal(g: np.random.Generator, shape, sigma: float) -> np.ndarray:
    z = g.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        z *= np.float32(sigma)
    return z


def _encode(z: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return z
    if dtype in ("bf16", "fp8_e4m3"):  # fp8 weights start as bf16; each side quantises them
        return f32_to_bf16_bits(z)
    raise ValueError(dtype)


def _store_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _stack(seed: int, tag: int, n: int, shape, sigma: float, dtype: str) -> np.ndarray:
    out = np.empty((n, *shape), dtype=_store_dtype(dtype))

    def one(i):
        out[i] = _encode(_normal(rng(seed, tag, i), shape, sigma), dtype)

    if n > 1 and int(np.prod(shape)) >= (1 << 20):
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(n)))
    else:
        for i in range(n):
            one(i)
    return out


def make_x(cfg: MoeConfig, step: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Activations of batch `step`: [T, H], N(0,1), in the config's activation dtype.

    Rows are drawn in chunks of X_CHUNK_ROWS with one child stream per chunk, so
    a batch of fewer rows is a prefix of the full batch of the same step.
    """
    T = cfg.T if T is None else T
    out = np.empty((T, cfg.H), dtype=_store_dtype(cfg.act))
    nchunk = (T + X_CHUNK_ROWS - 1) // X_CHUNK_ROWS

    def one(c):
        r0 = c * X_CHUNK_ROWS
        r1 = min(T, r0 + X_CHUNK_ROWS)
        z = _normal(rng(cfg.seed, TAG_X, step, c), (X_CHUNK_ROWS, cfg.H), 1.0)[: r1 - r0]
        out[r0:r1] = _encode(z, cfg.act)

    if nchunk > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunk)))
    else:
        one(0)
    return out


def make_logit_offset(cfg: MoeConfig) -> Optional[np.ndarray]:
    if cfg.offset_kind is None:
        return None
    g = rng(cfg.seed, TAG_OFF)
    if cfg.offset_kind == "normal":
        return g.standard_normal(cfg.E).astype(np.float32)
    if cfg.offset_kind == "zipf":
        ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
        p = ranks ** (-cfg.zipf_s)
        p /= p.sum()
        rank_of = rng(cfg.seed, TAG_PERM).permutation(cfg.E)  # expert e has rank rank_of[e] + 1
        return np.log(cfg.E * p[rank_of]).astype(np.float32)
    raise ValueError(cfg.offset_kind)


def make_bias0(cfg: MoeConfig) -> np.ndarray:
    if cfg.bias0_kind == "zero":
        return np.zeros(cfg.E, dtype=np.float32)
    if cfg.bias0_kind == "uniform":
        g = rng(cfg.seed, TAG_BIAS)
        return g.uniform(-cfg.bias0_range, cfg.bias0_range, cfg.E).astype(np.float32)
    raise ValueError(cfg.bias0_kind)


@dataclass
class LayerWeights:
    w_router: np.ndarray        # [E, H]   activation dtype (router stays bf16/fp32)
    w_gate_up: np.ndarray       # [E, 2I, H] gate rows [0, I), up rows [I, 2I)
    w_down: np.ndarray          # [E, H, I]
    ws_gate_up: np.ndarray      # [S, 2I, H]
    ws_down: np.ndarray         # [S, H, I]
    logit_offset: Optional[np.ndarray]  # [E] float32 or None
    bias0: np.ndarray           # [E] float32


def make_router(cfg: MoeConfig) -> LayerWeights:
    """The router part of make_weights (router weight, logit offset, initial bias; the
    same values), with empty expert tensors: for runs that draw expert weights elsewhere."""
    w_router = _encode(_normal(rng(cfg.seed, TAG_WR), (cfg.E, cfg.H), cfg.sigma), cfg.act)
    empty = np.empty((0,), dtype=_store_dtype(cfg.wgt))
    return LayerWeights(w_router, empty, empty, empty, empty, make_logit_offset(cfg), make_bias0(cfg))


def make_weights(cfg: MoeConfig) -> LayerWeights:
    s = cfg.seed
    w_router = _encode(_normal(rng(s, TAG_WR), (cfg.E, cfg.H), cfg.sigma), cfg.act)
    w_gu = _stack(s, TAG_WGU, cfg.E, (2 * cfg.I, cfg.H), cfg.sigma, cfg.wgt)
    w_d = _stack(s, TAG_WD, cfg.E, (cfg.H, cfg.I), cfg.sigma, cfg.wgt)
    ws_gu = _stack(s, TAG_SGU, cfg.S, (2 * cfg.I, cfg.H), cfg.sigma, cfg.wgt)
    ws_d = _stack(s, TAG_SD, cfg.S, (cfg.H, cfg.I), cfg.sigma, cfg.wgt)
    return LayerWeights(w_router, w_gu, w_d, ws_gu, ws_d, make_logit_offset(cfg), make_bias0(cfg))


def make_scores(seed: int, T: int, E: int, kind: str = "uniform") -> np.ndarray:
    """fp32 affinities in (0, 1) for routing-only checks.

    kind "uniform": U(0,1) float32 (ties essentially absent);
    kind "ties": multiples of 1/8, so group sums and top-k selections tie often;
    kind "zeros": contains +0.0 and -0.0 entries mixed with multiples of 1/4.
    """
    g = rng(seed, TAG_SCORES, T, E)
    if kind == "uniform":
        return g.random((T, E), dtype=np.float32)
    if kind == "ties":
        return (g.integers(1, 8, (T, E)) / 8.0).astype(np.float32)
    if kind == "zeros":
        v = (g.integers(0, 4, (T, E)) / 4.0).astype(np.float32)
        neg0 = (v == 0) & (g.random((T, E)) < 0.5)
        v[neg0] = np.float32(-0.0)
        return v
    raise ValueError(kind)
