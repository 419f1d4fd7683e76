"""Pins of the oracle's SwiGLU experts and FP8 codec/GEMM."""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from oracle import fp8 as ofp8
from workloads.inputs import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- SwiGLU
def test_swiglu_closed_form_identity_weights():
    """W_g = 2 I, W_u = I, W_d = I gives y = silu(2x) * x = 2x * expit(2x) * x;
    swapping gate and up would give silu(x) * 2x instead."""
    n = 16
    x = rng(1, 1).standard_normal((10, n))
    eye = np.eye(n)
    y = oracle.swiglu(x, np.concatenate([2 * eye, eye]), eye)
    np.testing.assert_allclose(y, 2 * x * expit(2 * x) * x, rtol=1e-14, atol=1e-300)


def test_swiglu_matches_torch_float64():
    H, I = 48, 40
    g = rng(2, 1)
    x = g.standard_normal((17, H))
    wgu = g.standard_normal((2 * I, H)) * 0.1
    wd = g.standard_normal((H, I)) * 0.1
    xt, wgut, wdt = (torch.from_numpy(a) for a in (x, wgu, wd))
    ref = (torch.nn.functional.silu(xt @ wgut[:I].T) * (xt @ wgut[I:].T)) @ wdt.T
    np.testing.assert_allclose(oracle.swiglu(x, wgu, wd), ref.numpy(), rtol=1e-12, atol=1e-14)


def test_shared_experts_sum_and_empty():
    H, I = 16, 8
    g = rng(3, 1)
    x = g.standard_normal((9, H))
    wgu = g.standard_normal((2, 2 * I, H))
    wd = g.standard_normal((2, H, I))
    y = oracle.shared_ffn(x, wgu, wd)
    np.testing.assert_allclose(y, oracle.swiglu(x, wgu[0], wd[0]) + oracle.swiglu(x, wgu[1], wd[1]),
                               rtol=1e-14)
    assert (oracle.shared_ffn(x, wgu[:0], wd[:0]) == 0).all()


def test_routed_ffn_uses_each_segments_expert():
    H, I, E = 8, 4, 3
    g = rng(4, 1)
    wgu = g.standard_normal((E, 2 * I, H))
    wd = g.standard_normal((E, H, I))
    xp = g.standard_normal((7, H))
    offsets = np.array([0, 2, 2, 7])
    y = oracle.routed_ffn(xp, offsets, wgu, wd)
    np.testing.assert_allclose(y[:2], oracle.swiglu(xp[:2], wgu[0], wd[0]))
    np.testing.assert_allclose(y[2:], oracle.swiglu(xp[2:], wgu[2], wd[2]))


# ---------------------------------------------------------------- FP8 codec
def test_e4m3_hand_points():
    with open(os.path.join(GOLDEN, "e4m3_points.json")) as f:
        pts = json.load(f)["points"]
    v = np.array([p[0] for p in pts])
    codes = np.array([p[1] for p in pts])
    assert (ofp8.e4m3_encode(v) == codes).all()


def test_e4m3_every_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = ofp8.e4m3_decode(codes)
    assert (ofp8.e4m3_encode(vals) == codes).all()
    assert np.isnan(ofp8.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert ofp8.e4m3_decode(np.array([0x7E], np.uint8))[0] == 448.0


def test_e4m3_matches_torch_conversion_in_range():
    """torch's float8_e4m3fn cast (round to nearest even) on a dense fp32 sweep of
    the finite range, including every midpoint between neighbouring codes."""
    mags = ofp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    sweep = np.concatenate([np.linspace(0, 448, 200001), mags, mids,
                            np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
                            np.nextafter(mids.astype(np.float32), np.float32(0))]).astype(np.float32)
    sweep = np.concatenate([sweep, -sweep])
    ref = torch.from_numpy(sweep).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ofp8.e4m3_encode(sweep) == ref).all()


def test_e4m3_saturates():
    v = np.array([449.0, 463.9, 480.0, 1e6, np.float32(3e38), -500.0], np.float32)
    assert ofp8.e4m3_encode(v).tolist() == [0x7E] * 5 + [0xFE]


def test_quantize_rows_error_bound_and_tile_max():
    g = rng(5, 1)
    v = (g.standard_normal((6, 512)) * np.exp(g.standard_normal((6, 1)) * 3)).astype(np.float32)
    v[2, 128:256] = 0.0          # an all-zero tile keeps scale 1
    q, sc = ofp8.quantize_rows_1x128(v)
    assert q.shape == v.shape and sc.shape == (6, 4)
    assert sc[2, 1] == 1.0 and (q[2, 128:256] == 0).all()
    deq = ofp8.e4m3_decode(q) * np.repeat(sc, 128, axis=1)
    rel = np.abs(deq - v) / np.maximum(np.abs(v), 2.0 ** -6 * np.repeat(sc, 128, axis=1).astype(np.float64))
    assert rel.max() <= 2.0 ** -4 + 1e-6      # half an ulp of a 3-bit mantissa
    mx = (q & 0x7F).reshape(6, 4, 128).max(axis=2)
    assert (mx[sc != 1.0] == 0x7E).all()       # every tile's largest value maps to 448


def test_fp8_matmul_equals_dequantised_product():
    g = rng(6, 1)
    a = g.standard_normal((9, 384)).astype(np.float32)
    w = (g.standard_normal((256, 384)) * 0.02).astype(np.float32)
    qa, sa = ofp8.quantize_rows_1x128(a)
    qw, sw = ofp8.quantize_blocks_128x128(w)
    assert sw.shape == (2, 3)
    A = ofp8.e4m3_decode(qa) * np.repeat(sa, 128, axis=1)
    W = ofp8.e4m3_decode(qw) * np.repeat(np.repeat(sw, 128, axis=0), 128, axis=1)
    np.testing.assert_allclose(ofp8.fp8_matmul(qa, sa, qw, sw), A @ W.T, rtol=1e-12, atol=1e-12)
    # and it approximates the unquantised product to FP8 accuracy
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    err = np.abs(ofp8.fp8_matmul(qa, sa, qw, sw) - ref).max() / np.abs(ref).max()
    assert err < 0.06


@pytest.mark.parametrize("shape", [(128, 256), (384, 128)])
def test_quantize_blocks_scale_layout(shape):
    g = rng(7, shape[0])
    w = g.standard_normal(shape).astype(np.float32)
    w[:128, :128] *= 100.0      # one hot block must not change the others' scales
    q, sc = ofp8.quantize_blocks_128x128(w)
    assert sc.shape == (shape[0] // 128, shape[1] // 128)
    assert sc[0, 0] == np.float32(np.abs(w[:128, :128]).max() / np.float32(448))
    if shape[1] > 128:
        assert sc[0, 1] == np.float32(np.abs(w[:128, 128:256]).max() / np.float32(448))
