"""GPU parity at the V3-like layer shapes (hidden 7168, 256 routed experts in 8 groups,
at most 4 groups per token, top-8, 1 shared expert, intermediate 2048, gate scale 2.5,
bf16), in the launch configuration the benchmark times.

Prefill (T=16384) and decode (T=128) share the weights.  Routing, counts, the
permutation and the bias update are checked over the whole batch (bit-exact,
teacher-forced on the GPU's fp32 scores; own-score index flips only at oracle
near-ties below 1e-5).  Expert outputs are checked on samples the fp64 oracle can
afford: whole segments of a few experts (y_perm), the shared expert on sampled
tokens, and the full layer output on 256 sampled tokens, among them the last 16 of the batch
and tokens of the largest expert segment (every token at decode size; normwise 2e-2)."""
import numpy as np
import pytest
import torch

import oracle
from biased_top_routing_amd import _lib as L
from biased_top_routing_amd.runner import MoeLayerGPU, to_device
from gpu_util import dev_f32, host, rel_inf, sample_tokens, say
from workloads import V3_PREFILL
from oracle.layer import decode_act
from workloads.inputs import f32_to_bf16_bits, make_weights, make_x, rng

pytestmark = pytest.mark.gpu

GAP = 1e-5


@pytest.fixture(scope="module")
def v3():
    say("v3: generating weights (22.5 GB bf16)")
    w = make_weights(V3_PREFILL)
    say("v3: uploading")
    layer = MoeLayerGPU(V3_PREFILL, w)
    torch.cuda.synchronize()
    return w, layer


def _run(c, w, layer, T, step):
    if layer.T != T:
        layer.alloc(T)
    xh = make_x(c, step, T=T)
    bias_h = w.bias0.copy()
    bias = dev_f32(bias_h)
    say(f"v3 forward T={T}")
    y = layer.forward(to_device(xh), bias, gamma=c.gamma)
    torch.cuda.synchronize()
    return xh, bias_h, host(bias), host(y)


def _check_routing(c, T, w, layer, xh, bias_h, bias_next):
    s_gpu = host(layer.scores)
    idx = host(layer.topk_idx)
    # teacher-forced: the oracle routes the GPU's own fp32 scores
    idx_o, w_o = oracle.route(s_gpu, bias_h, c.G, c.M, c.k, c.group_topr, c.route_scale)
    assert (idx == idx_o).all()
    np.testing.assert_allclose(host(layer.topk_w), w_o, rtol=2e-6, atol=1e-7)
    counts, offsets, perm, inv = oracle.dispatch(idx, c.E)
    assert (host(layer.counts) == counts).all()
    assert (host(layer.offsets) == offsets).all()
    assert (host(layer.perm) == perm).all()
    assert (host(layer.inv) == inv).all()
    exp_b = oracle.update_bias(bias_h, counts, T, c.k, c.gamma)
    assert (bias_next.view(np.uint32) == exp_b.view(np.uint32)).all()
    # own scores: fp64 oracle affinity; index flips only at near-ties
    say("v3: oracle affinity over the batch")
    s_ora = oracle.affinity(oracle.decode_act(xh).astype(np.float64),
                            oracle.decode_act(w.w_router).astype(np.float64), w.logit_offset)
    assert np.abs(s_gpu - s_ora).max() < 1e-4
    ref_idx, _ = oracle.route(s_ora, bias_h, c.G, c.M, c.k, c.group_topr, c.route_scale)
    gk, gm = oracle.route_diagnostics(s_ora, bias_h, c.G, c.M, c.k, c.group_topr)
    # the selected set may differ only at a near-tie (slot order within a set may differ
    # wherever two selected scores are within rounding of each other)
    bad = (np.sort(ref_idx, axis=1) != np.sort(idx, axis=1)).any(axis=1)
    assert ((gk[bad] < GAP) | (gm[bad] < GAP)).all()
    say(f"  near-tie index flips: {int(bad.sum())} of {T}")
    return s_ora, idx, offsets, perm


def _check_outputs(c, w, layer, xh, s_ora, idx, offsets, perm, y, n_tok, experts):
    # whole segments of a few experts
    yp = layer.y_perm
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        say(f"  expert {e}: {hi - lo} rows")
        ref = oracle.swiglu(oracle.decode_act(xh[perm[lo:hi] // c.k]), oracle.decode_act(w.w_gate_up[e]),
                            oracle.decode_act(w.w_down[e]))
        assert rel_inf(host(yp[lo:hi]), ref) < 2e-2
    # shared expert and full layer output on sampled tokens (the last rows of the batch
    # and tokens of the largest expert segment among them)
    rows = sample_tokens(len(xh), idx, n_tok, 7)
    ref_sh = oracle.shared_ffn(oracle.decode_act(xh[rows]), [oracle.decode_act(a) for a in w.ws_gate_up],
                               [oracle.decode_act(a) for a in w.ws_down])
    assert rel_inf(host(layer.y_shared)[rows], ref_sh) < 2e-2
    sel = np.take_along_axis(s_ora[rows].astype(np.float64), idx[rows].astype(np.int64), 1)
    w_rows = c.route_scale * sel / sel.sum(1, keepdims=True)
    say(f"  sampled layer output on {n_tok} tokens")
    ref_y = oracle.sampled_forward(c, xh[rows], idx[rows], w_rows, w)
    err = rel_inf(y[rows], ref_y)
    say(f"  sampled y err {err:.2e}")
    assert err < 2e-2


def test_v3_prefill_full_size(v3):
    w, layer = v3
    c = V3_PREFILL
    xh, bias_h, bias_next, y = _run(c, w, layer, c.T, 0)
    s_ora, idx, offsets, perm = _check_routing(c, c.T, w, layer, xh, bias_h, bias_next)
    _check_outputs(c, w, layer, xh, s_ora, idx, offsets, perm, y, n_tok=256,
                   experts=(0, 131, 255, int(np.argmax(np.diff(offsets)))))


def test_v3_decode_full_size(v3):
    w, layer = v3
    c = V3_PREFILL.with_(name="v3_decode_bf16", T=128)
    xh, bias_h, bias_next, y = _run(c, w, layer, c.T, 3)
    s_ora, idx, offsets, perm = _check_routing(c, c.T, w, layer, xh, bias_h, bias_next)
    _check_outputs(c, w, layer, xh, s_ora, idx, offsets, perm, y, n_tok=c.T,
                   experts=(int(idx[0, 0]), int(np.argmax(np.diff(offsets)))))


def test_v3_prefill_gather_bit_exact(v3):
    """Dispatch without the row copy and the gate/up GEMM gathering its rows from x
    (the benchmark's path) give the materialised path's indices and outputs bit for bit."""
    w, layer = v3
    c = V3_PREFILL
    xh, _, _, _ = _run(c, w, layer, c.T, 0)
    x = to_device(xh)
    counts, offsets = torch.empty_like(layer.counts), torch.empty_like(layer.offsets)
    perm, inv = torch.empty_like(layer.perm), torch.empty_like(layer.inv)
    say("v3: dispatch without x_perm")
    L.moe_dispatch(layer.cfg, layer.topk_idx, None, counts, offsets, perm, inv, None, None, layer.ws_dispatch)
    for a, b in ((counts, layer.counts), (offsets, layer.offsets), (perm, layer.perm), (inv, layer.inv)):
        assert torch.equal(a, b)
    y_perm, y_shared = torch.empty_like(layer.y_perm), torch.empty_like(layer.y_shared)
    ws = torch.empty_like(layer.ws_ffn)
    say("v3: gathered expert FFN")
    L.moe_expert_ffn_gather(layer.cfg, x, perm, offsets, layer.weights, y_perm, y_shared, ws)
    torch.cuda.synchronize()
    assert torch.equal(y_perm.view(torch.int16), layer.y_perm.view(torch.int16))
    assert torch.equal(y_shared.view(torch.int16), layer.y_shared.view(torch.int16))


def test_v3_prefill_backward_full_size(v3):
    """The layer backward at the full V3-like size (the training step's shape), on
    samples the fp64 oracle can afford: two whole experts' weight gradients, the
    complete input gradient of sampled tokens (8 routed experts, the shared one,
    the router and the balance term), d_topk_w of those tokens, dW_router (fp64
    from the GPU's own d_topk_w) and the balance loss."""
    from oracle.backward import gate_backward, seq_balance_loss, swiglu_backward
    w, layer = v3
    c = V3_PREFILL
    alpha, seq_len = 1e-3, 4096
    xh, _, _, _ = _run(c, w, layer, c.T, 0)   # forward (with the bias update: the routing is what counts)
    x = to_device(xh)
    dyh = f32_to_bf16_bits(rng(31, c.T).normal(size=(c.T, c.H)).astype(np.float32))
    say("v3: backward")
    layer.backward(x, to_device(dyh), alpha, seq_len)
    torch.cuda.synchronize()
    idx = host(layer.topk_idx).astype(np.int64)
    dyf = decode_act(dyh).astype(np.float64)
    say("v3: oracle affinities and balance term")
    x64 = decode_act(xh).astype(np.float64)
    wr = decode_act(w.w_router).astype(np.float64)
    logits = x64 @ wr.T + (0.0 if w.logit_offset is None else np.asarray(w.logit_offset, np.float64))
    s = 1.0 / (1.0 + np.exp(-logits))
    loss, ds_bal = seq_balance_loss(s, idx, c.k, seq_len, alpha)
    assert abs(float(host(layer.loss_bal)[0]) - loss) <= 1e-4 * loss
    s_sel = np.take_along_axis(s, idx, axis=1)
    gates = c.route_scale * s_sel / s_sel.sum(axis=1, keepdims=True)
    # dW_router from the GPU's d_topk_w
    dw_gpu = host(layer.d_topk_w).astype(np.float64)
    ds = ds_bal.copy()
    np.put_along_axis(ds, idx, np.take_along_axis(ds, idx, axis=1) + gate_backward(s_sel, dw_gpu, c.route_scale),
                      axis=1)
    dlogit = ds * s * (1.0 - s)
    err = rel_inf(host(layer.g_w_router), dlogit.T @ x64)
    say(f"  dW_router err {err:.2e}")
    assert err < 2e-2
    # sampled tokens: everything from scratch
    rows = np.sort(rng(41, 6).choice(c.T, 6, replace=False))
    wsgu = decode_act(w.ws_gate_up[0]).astype(np.float64)
    wsd = decode_act(w.ws_down[0]).astype(np.float64)
    dx_ref = np.zeros((len(rows), c.H))
    dw_ref = np.zeros((len(rows), c.k))
    for n, t in enumerate(rows):
        xt = x64[t:t + 1]
        for j in range(c.k):
            e = idx[t, j]
            wgu, wd = decode_act(w.w_gate_up[e]).astype(np.float64), decode_act(w.w_down[e]).astype(np.float64)
            dw_ref[n, j] = float((dyf[t] * oracle.swiglu(xt, wgu, wd)[0]).sum())
            dx_ref[n] += swiglu_backward(xt, wgu, wd, gates[t, j] * dyf[t:t + 1])[0][0]
        dx_ref[n] += swiglu_backward(xt, wsgu, wsd, dyf[t:t + 1])[0][0]
    ds_rows = ds_bal[rows].copy()
    np.put_along_axis(ds_rows, idx[rows], np.take_along_axis(ds_rows, idx[rows], axis=1) +
                      gate_backward(s_sel[rows], dw_ref, c.route_scale), axis=1)
    dx_ref += (ds_rows * s[rows] * (1.0 - s[rows])) @ wr
    e_dw = rel_inf(dw_gpu[rows], dw_ref)
    e_dx = rel_inf(host(layer.dx)[rows], dx_ref)
    say(f"  sampled d_topk_w err {e_dw:.2e}, dx err {e_dx:.2e}")
    assert e_dw < 2e-2 and e_dx < 2e-2
    # two whole experts' weight gradients (the two smallest non-empty segments)
    counts = np.bincount(idx.reshape(-1), minlength=c.E)
    for e in np.argsort(np.where(counts > 0, counts, 1 << 30), kind="stable")[:2]:
        t_of, j_of = np.nonzero(idx == e)
        say(f"  expert {e}: {len(t_of)} rows")
        _, dwgu, dwd, _ = swiglu_backward(x64[t_of], decode_act(w.w_gate_up[e]).astype(np.float64),
                                          decode_act(w.w_down[e]).astype(np.float64),
                                          gates[t_of, j_of][:, None] * dyf[t_of])
        e1 = rel_inf(host(layer.g_w_gate_up[e]), dwgu)
        e2 = rel_inf(host(layer.g_w_down[e]), dwd)
        say(f"    dW_gate_up err {e1:.2e}, dW_down err {e2:.2e}")
        assert e1 < 2e-2 and e2 < 2e-2


def test_v3_prefill_saved_backward_bit_exact(v3):
    """At the full V3-like size, the training step that keeps g, u in the forward pass
    (moe_expert_ffn_save + moe_expert_ffn_backward_saved) gives the same forward output
    and the same gradients, bit for bit, as the one that recomputes them."""
    w, layer = v3
    c = V3_PREFILL
    layer.save_gu = True
    layer.alloc(c.T)                                  # buffers for g, u
    xh = make_x(c, 0)
    x = to_device(xh)
    dy = to_device(f32_to_bf16_bits(rng(33, c.T).normal(size=(c.T, c.H)).astype(np.float32)))
    bias = dev_f32(w.bias0)
    keys = ["dx", "dx_shared", "g_w_gate_up", "g_w_down", "g_ws_gate_up", "g_ws_down", "g_w_router", "loss_bal"]
    iview = lambda t: t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)
    kept = None
    for save in (True, False):
        layer.save_gu = save
        say(f"v3: forward + backward, g and u {'kept' if save else 'recomputed'}")
        y = layer.forward(x, bias)
        layer.backward(x, dy, 1e-3, 4096)
        torch.cuda.synchronize()
        if save:                                      # one copy (the weight gradients are 45 GB of fp32)
            kept = {"y": y.clone(), **{k: getattr(layer, k).clone() for k in keys}}
    layer.save_gu = False
    assert torch.equal(iview(kept["y"]), iview(y)), "y differs"
    for k in keys:
        assert torch.equal(iview(kept[k]), iview(getattr(layer, k))), f"{k} differs"
