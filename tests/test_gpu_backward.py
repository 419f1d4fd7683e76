"""GPU parity of the layer backward (moe_combine_backward -> moe_expert_ffn_backward
-> moe_route_backward -> moe_dispatch_backward) against the fp64 backward oracle,
teacher-forced on the GPU's own expert choice.

* dy_perm = bf16(fl32(w * dy)) bit for bit (the same fp32 product and rounding
  written independently in numpy).
* d_topk_w, dx, every expert's dW_gate_up and dW_down, the shared experts'
  gradients, dW_router and dx_router normwise against the oracle: bf16 operands
  (x, weights, dy, the recomputed g, u, h, dgu and dlogit are each rounded to
  bf16 once) with fp32 accumulation give ~2^-8 relative error; the bound is 2e-2
  per tensor and per expert.  Empty experts have exactly zero gradients.
* The balance-loss value to 1e-4 relative (fp32 sums over the sequence).
* Two calls give identical bits (every reduction has a fixed order).
Cases: 16 experts with K = E below one 64-slice (router GEMMs) and a 128-token
sequence length; two shared experts with H and I off the 256-column tile grid;
a Zipf-skewed layer without shared experts and without the balance loss (empty
experts, ragged segments); one sequence over the whole batch."""
import numpy as np
import pytest
import torch

from biased_top_routing_amd.runner import MoeLayerGPU, to_device
from gpu_util import host, rel_inf, say
from oracle.backward import backward_from_routing
from oracle.layer import decode_act
from workloads import MID
from workloads.inputs import f32_to_bf16_bits, make_weights, make_x, rng

pytestmark = pytest.mark.gpu

TOL = 2e-2
CASES = {
    "e16_seq128": (MID.with_(T=512, H=256, E=16, G=4, M=2, k=4, S=1, I=256), 0.1, 128),
    "s2_ragged_tiles": (MID.with_(T=1000, H=384, E=64, I=384, S=2), 0.05, 250),
    "zipf_no_shared_no_loss": (MID.with_(T=300, H=256, E=64, I=128, S=0), 0.0, 0),
    "one_sequence": (MID.with_(T=256, H=512, E=32, G=4, M=2, k=4, S=1, I=128), 0.2, 0),
}


def _f64(a):
    return decode_act(a).astype(np.float64)


def _bits(t):
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    c, alpha, seq_len = CASES[name]
    w = make_weights(c)
    xh = make_x(c)
    dyh = f32_to_bf16_bits(rng(99, c.T).normal(size=(c.T, c.H)).astype(np.float32))
    say(f"backward {name}: forward + backward on the GPU")
    layer = MoeLayerGPU(c, w)
    x = to_device(xh)
    dy = to_device(dyh)
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    layer.forward(x, bias)
    layer.backward(x, dy, alpha, seq_len)
    torch.cuda.synchronize()
    first = {k: _bits(getattr(layer, k)).copy() for k in ("dx", "g_w_gate_up", "g_w_down", "g_w_router")}
    layer.backward(x, dy, alpha, seq_len)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert (v == _bits(getattr(layer, k))).all(), f"{k} differs between two calls"

    idx = host(layer.topk_idx).astype(np.int64)
    inv = host(layer.inv).astype(np.int64)
    tw = host(layer.topk_w)
    # dy_perm: the same fp32 product and bf16 rounding
    dy32 = decode_act(dyh)
    exp = f32_to_bf16_bits((tw[:, :, None] * dy32[:, None, :]).astype(np.float32))   # [T, k, H]
    got = _bits(layer.dy_perm).view(np.uint16)
    assert (got[inv.reshape(-1)] == exp.reshape(-1, c.H)).all(), "dy_perm"

    say(f"backward {name}: fp64 oracle")
    ws_gu = [_f64(a) for a in w.ws_gate_up] if c.S else None
    ws_d = [_f64(a) for a in w.ws_down] if c.S else None
    o = backward_from_routing(_f64(xh), _f64(w.w_router), w.logit_offset, _f64(w.w_gate_up), _f64(w.w_down),
                              ws_gu, ws_d, idx, _f64(dyh), c.route_scale, alpha, seq_len)
    errs = {"d_topk_w": rel_inf(host(layer.d_topk_w), o["dw"]),
            "dx": rel_inf(host(layer.dx), o["dx"]),
            "dw_router": rel_inf(host(layer.g_w_router), o["dw_router"]),
            "dx_router": rel_inf(host(layer.dx_router), o["dlogit"] @ _f64(w.w_router))}
    gwu, gwd = host(layer.g_w_gate_up), host(layer.g_w_down)
    counts = np.bincount(idx.reshape(-1), minlength=c.E)
    for e in range(c.E):
        if counts[e] == 0:
            assert not gwu[e].any() and not gwd[e].any(), f"expert {e} has no rows but a gradient"
            continue
        errs[f"dw_gate_up[{e}]"] = rel_inf(gwu[e], o["dw_gate_up"][e])
        errs[f"dw_down[{e}]"] = rel_inf(gwd[e], o["dw_down"][e])
    if c.S:
        errs["dws_gate_up"] = rel_inf(host(layer.g_ws_gate_up), o["dws_gate_up"])
        errs["dws_down"] = rel_inf(host(layer.g_ws_down), o["dws_down"])
    worst = max(errs, key=errs.get)
    say(f"backward {name}: worst {worst} {errs[worst]:.2e}; dx {errs['dx']:.2e}, dW_r {errs['dw_router']:.2e}")
    bad = {k: v for k, v in errs.items() if not v < TOL}
    assert not bad, bad
    loss = float(host(layer.loss_bal)[0])
    if alpha:
        assert abs(loss - o["loss_bal"]) <= 1e-4 * abs(o["loss_bal"]), (loss, o["loss_bal"])
    else:
        assert loss == 0.0


@pytest.mark.parametrize("name", ["s2_ragged_tiles", "zipf_no_shared_no_loss"])
def test_saved_gate_up_matches_recompute(name):
    """A forward pass that keeps g, u (moe_expert_ffn_save) gives the same y as one that
    does not, and the backward pass from the kept g, u (moe_expert_ffn_backward_saved)
    the same gradients as the one that recomputes them, bit for bit (the same GEMM
    computes both, in the same order)."""
    c, alpha, seq_len = CASES[name]
    w = make_weights(c)
    xh = make_x(c)
    dyh = f32_to_bf16_bits(rng(98, c.T).normal(size=(c.T, c.H)).astype(np.float32))
    say(f"saved g/u {name}")
    layer = MoeLayerGPU(c, w, save_gu=True)
    x, dy = to_device(xh), to_device(dyh)
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    y_saved = _bits(layer.forward(x, bias)).copy()
    layer.backward(x, dy, alpha, seq_len)
    torch.cuda.synchronize()
    keys = ["dx", "dx_shared", "dx_perm", "g_w_gate_up", "g_w_down", "g_ws_gate_up", "g_ws_down", "g_w_router",
            "loss_bal"]
    saved = {k: _bits(getattr(layer, k)).copy() for k in keys if getattr(layer, k) is not None}
    layer.save_gu = False                      # same buffers, the recomputing entry points
    y_plain = _bits(layer.forward(x, bias)).copy()
    layer.backward(x, dy, alpha, seq_len)
    torch.cuda.synchronize()
    assert (y_saved == y_plain).all(), "y differs with and without keeping g, u"
    for k, v in saved.items():
        assert (v == _bits(getattr(layer, k))).all(), f"{k}: saved g, u and recomputation differ"


def test_save_by_phase():
    """moe_expert_ffn_save run as its two phases (gate/up, then down) writes the same g, u,
    y_perm and y_shared as one call, and the down phase leaves the kept g, u untouched."""
    from biased_top_routing_amd import _lib as L
    c, _, _ = CASES["s2_ragged_tiles"]
    w = make_weights(c)
    xh = make_x(c)
    layer = MoeLayerGPU(c, w, save_gu=True)
    x = to_device(xh)
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    layer.forward(x, bias)
    torch.cuda.synchronize()
    whole = {k: _bits(getattr(layer, k)).copy() for k in ("g", "u", "gs", "us", "y_perm", "y_shared")}
    for k in ("g", "u", "gs", "us", "y_perm", "y_shared"):
        getattr(layer, k).zero_()
    layer.expert_ffn(x, L.MOE_FFN_GATE_UP)
    torch.cuda.synchronize()
    kept = {k: _bits(getattr(layer, k)).copy() for k in ("g", "u", "gs", "us")}
    for k in ("g", "u", "gs", "us"):
        getattr(layer, k).fill_(1.0)                  # the down phase must not touch them
    layer.expert_ffn(x, L.MOE_FFN_DOWN)
    torch.cuda.synchronize()
    for k in ("g", "u", "gs", "us"):
        assert (kept[k] == whole[k]).all(), f"{k} from the gate/up phase differs"
        assert (getattr(layer, k) == 1.0).all(), f"the down phase wrote {k}"
    for k in ("y_perm", "y_shared"):
        assert (_bits(getattr(layer, k)) == whole[k]).all(), f"{k} by phases differs"
