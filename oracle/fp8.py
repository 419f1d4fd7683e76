"""Oracle: fine-grained FP8 (E4M3) quantisation and the block-scaled GEMM.

TEST INFRASTRUCTURE (see the package docstring).

What the pages fix (qwbw.cn essay, FP8 part of the training-infrastructure
section; DeepSeek-V3 Technical Report：中英对照解读, §6 FP8 Training):
* E4M3 for every FP8 tensor;
* one scale per 1x128 tile of an activation row and per 128x128 block of a
  weight, so an outlier only widens the range of its own tile;
* low-precision products are promoted to full-precision accumulation every
  128 elements of K.

Readings: the format is OCP E4M3FN (bias 7, no infinities, largest finite
value 448, code 0x7F/0xFF is NaN); encoding rounds to nearest with ties to the
even code and saturates at +-448; a tile's scale is sc = fl32(amax / 448)
(sc = 1 for an all-zero tile) and a value v is stored as encode(fl32(v / sc)).
The GEMM sums code products exactly within each 128-wide K chunk (they fit in
fp64 exactly), multiplies the chunk sum by both scales and accumulates in fp64.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64
E4M3_MAX = 448.0
TILE = 128


def e4m3_decode(codes) -> np.ndarray:
    """Real value of each E4M3FN code, from the bit fields (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# magnitudes of the 127 non-negative finite codes 0x00..0x7E, increasing with the code
_MAGS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3FN code (ties to the even code), saturating at +-448.  NaN input is undefined."""
    v = np.asarray(v, F64)
    a = np.abs(v)
    hi = np.searchsorted(_MAGS, a, side="left")          # _MAGS[hi-1] < a <= _MAGS[hi]
    hi = np.minimum(hi, len(_MAGS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= _MAGS[-1], len(_MAGS) - 1, code)   # saturate
    code = np.where(a == _MAGS[hi], hi, code)                # exact hit
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _scale_of(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, F32)
    sc = (amax / F32(E4M3_MAX)).astype(F32)
    return np.where(amax == 0, F32(1.0), sc).astype(F32)


def quantize_rows_1x128(v) -> tuple:
    """Per-row, per-128-column tiles.  v [R, K] real values, K % 128 == 0.

    Returns codes uint8 [R, K] and scales float32 [R, K/128].
    """
    v = np.asarray(v, F32)
    R, K = v.shape
    t = v.reshape(R, K // TILE, TILE)
    sc = _scale_of(np.abs(t).max(axis=2))
    q = e4m3_encode((t / sc[:, :, None]).astype(F32))
    return q.reshape(R, K), sc


def quantize_blocks_128x128(w) -> tuple:
    """128 x 128 blocks of a weight w [N, K] (N, K multiples of 128).

    Returns codes uint8 [N, K] and scales float32 [N/128, K/128].
    """
    w = np.asarray(w, F32)
    N, K = w.shape
    b = w.reshape(N // TILE, TILE, K // TILE, TILE)
    sc = _scale_of(np.abs(b).max(axis=(1, 3)))
    q = e4m3_encode((b / sc[:, None, :, None]).astype(F32))
    return q.reshape(N, K), sc


# value of every byte, for decoding large arrays by lookup (the same values e4m3_decode gives)
_DECODE = e4m3_decode(np.arange(256, dtype=np.uint8))


def fp8_matmul(qa, sa, qw, sw) -> np.ndarray:
    """out[r, n] = sum_c (sum_{k in chunk c} a_code*w_code) * sa[r, c] * sw[n // 128, c]  (fp64)."""
    A = _DECODE[np.asarray(qa, np.uint8)]
    W = _DECODE[np.asarray(qw, np.uint8)]
    R, K = A.shape
    N = W.shape[0]
    out = np.zeros((R, N), F64)
    sa = np.asarray(sa, F64)
    sw = np.asarray(sw, F64)
    for c in range(K // TILE):
        part = A[:, c * TILE:(c + 1) * TILE] @ W[:, c * TILE:(c + 1) * TILE].T   # exact in fp64
        out += part * sa[:, c:c + 1] * np.repeat(sw[:, c], TILE)[None, :]
    return out
