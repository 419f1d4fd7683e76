"""Pins of the oracle's whole-layer forward and of the workload generators."""
import numpy as np
import torch

import oracle
from workloads import MID, TINY, V3_FP8
from workloads.inputs import make_bias0, make_logit_offset, make_weights, make_x


def test_single_expert_layer_is_dense_swiglu():
    """E = 1, k = 1, no shared expert, scale 1: the layer is one dense SwiGLU
    (gate = s/s = 1), computed here with torch's float64 silu and matmul."""
    cfg = TINY.with_(E=1, G=1, M=1, k=1, S=0, group_topr=1)
    w = make_weights(cfg)
    x = make_x(cfg)
    out = oracle.layer_forward(cfg, x, w, w.bias0)
    xt = torch.from_numpy(x.astype(np.float64))
    gu = torch.from_numpy(w.w_gate_up[0].astype(np.float64))
    wd = torch.from_numpy(w.w_down[0].astype(np.float64))
    ref = (torch.nn.functional.silu(xt @ gu[:cfg.I].T) * (xt @ gu[cfg.I:].T)) @ wd.T
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-15)
    assert (out["counts"] == [cfg.T]).all()


def test_tiny_layer_invariants_and_sampled_path():
    cfg = TINY
    w = make_weights(cfg)
    x = make_x(cfg)
    out = oracle.layer_forward(cfg, x, w, w.bias0)
    assert out["idx"].shape == (cfg.T, cfg.k)
    assert np.abs(out["w"].sum(1) - cfg.route_scale).max() < 1e-12
    assert out["counts"].sum() == cfg.T * cfg.k
    rows = np.array([0, 5, 77, 255])
    ys = oracle.sampled_forward(cfg, x[rows], out["idx"][rows], out["w"][rows], w)
    np.testing.assert_allclose(ys, out["y"][rows], rtol=1e-12, atol=1e-14)
    # the bias moved by exactly +-gamma
    d = out["bias_next"] - w.bias0
    assert np.allclose(np.abs(d), np.float32(1e-3))


def test_fp8_layer_close_to_unquantised():
    cfg = V3_FP8.with_(T=64, H=256, E=16, G=4, M=2, k=4, I=128, S=1)
    w = make_weights(cfg)
    x = make_x(cfg)
    b = np.zeros(cfg.E, np.float32)
    q = oracle.layer_forward(cfg, x, w, b)
    ref = oracle.layer_forward(cfg.with_(wgt="bf16"), x, w, b)
    assert (q["idx"] == ref["idx"]).all()          # routing stays in higher precision
    err = np.abs(q["y"] - ref["y"]).max() / np.abs(ref["y"]).max()
    assert 1e-4 < err < 0.15


def test_workload_generators_deterministic_and_prefix():
    a = make_x(MID, step=3, T=1500)
    b = make_x(MID, step=3)
    assert a.dtype == np.uint16 and (a == b[:1500]).all()
    assert not (make_x(MID, step=4, T=8) == b[:8]).all()
    w1 = make_weights(TINY)
    w2 = make_weights(TINY)
    assert (w1.w_gate_up == w2.w_gate_up).all() and w1.w_gate_up.dtype == np.float32


def test_zipf_offsets_span():
    """o_e = ln(E p_rank) with p_r proportional to r^-s: the hottest expert gets
    ln(E / H_{E,s}) and the coldest ln(E E^-s / H_{E,s})."""
    o = make_logit_offset(MID).astype(np.float64)
    Hs = (np.arange(1, 65) ** -1.1).sum()
    assert abs(o.max() - np.log(64 / Hs)) < 1e-6
    assert abs(o.min() - np.log(64 * 64 ** -1.1 / Hs)) < 1e-6
    assert len(set(np.round(o, 6))) == 64
    assert (make_bias0(MID) == 0).all()
