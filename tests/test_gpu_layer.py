"""GPU parity, tolerance part: combine, expert GEMMs and the whole layer.

Tolerances (normwise max relative error ||y - y_ref||_inf / ||y_ref||_inf against
the fp64 oracle): fp32 path 1e-4; bf16 path 2e-2.  The bf16 path rounds h,
y_perm, y_shared and y to bf16 (relative 2^-9 each) and accumulates in fp32, so
its expected error is well under 1%.  Routing on the full path is compared with
the rule that an index may differ only where the oracle's k-th/(k+1)-th score
gap (or its M-th/(M+1)-th group-score gap) is below 1e-5; outputs are compared
teacher-forced on the GPU's selection."""
import numpy as np
import pytest
import torch

import oracle
from biased_top_routing_amd import _lib as L
from biased_top_routing_amd.runner import MoeLayerGPU, to_device
from gpu_util import dev_f32, dev_i32, host, rel_inf, say
from workloads import MID, TINY, V3_PREFILL
from workloads.inputs import f32_to_bf16_bits, make_weights, make_x, rng

pytestmark = pytest.mark.gpu

GAP = 1e-5


def _bf16_dev(a_f32):
    return torch.from_numpy(f32_to_bf16_bits(a_f32).view(np.int16)).cuda().view(torch.bfloat16)


def _dec(bits):
    return oracle.decode_act(bits).astype(np.float64)


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_combine(act):
    T, E, k, H, S = 500, 16, 4, 256, 1
    say(f"combine {act} T={T} H={H}")
    cfg = L.make_cfg(T, H, E, 4, 2, k, S, 128, 2, 1.0, act, act)
    g = rng(11, 1)
    idx = np.argsort(-g.random((T, E)), axis=1)[:, :k].astype(np.int32)
    _, _, perm, inv = oracle.dispatch(idx, E)
    w = g.random((T, k)).astype(np.float32)
    yp = g.standard_normal((T * k, H)).astype(np.float32)
    ys = g.standard_normal((T, H)).astype(np.float32)
    if act == "bf16":
        yp_d, ys_d = _bf16_dev(yp), _bf16_dev(ys)
        yp_v, ys_v = _dec(f32_to_bf16_bits(yp)), _dec(f32_to_bf16_bits(ys))
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        tol = 2 ** -8
    else:
        yp_d, ys_d, yp_v, ys_v = dev_f32(yp), dev_f32(ys), yp, ys
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        tol = 1e-6
    L.moe_combine(cfg, yp_d, ys_d, dev_i32(inv), dev_f32(w), y)
    torch.cuda.synchronize()
    ref = oracle.combine(yp_v, ys_v, inv, w)
    assert rel_inf(host(y), ref) < tol


# Rows whose 16-byte chunk count leaves a last wavefront with fewer active lanes than k
# (0 < nchunk mod 64 < k), and a second pass over the row (nchunk > 1024): every slot
# of every chunk must still be added.
COMBINE_TAIL_CASES = [
    # (act, T, H, E, G, M, k)
    ("bf16", 37, 576, 32, 4, 2, 16),     # 72 chunks: 8 lanes in the last wavefront
    ("bf16", 9, 8256, 32, 4, 2, 16),     # 1032 chunks: a second pass of 8 lanes
    ("f32", 41, 68, 32, 4, 4, 24),       # 17 chunks
    ("f32", 50, 12, 8, 2, 2, 4),         # 3 chunks
]


@pytest.mark.parametrize("act,T,H,E,G,M,k", COMBINE_TAIL_CASES)
def test_combine_ragged_row_tail(act, T, H, E, G, M, k):
    say(f"combine tail {act} T={T} H={H} k={k}")
    cfg = L.make_cfg(T, H, E, G, M, k, 1, 128 if act == "bf16" else 4, 2, 1.0, act, act)
    g = rng(12, H, k)
    idx = np.argsort(-g.random((T, E)), axis=1)[:, :k].astype(np.int32)
    _, _, perm, inv = oracle.dispatch(idx, E)
    w = (g.random((T, k)) + 0.5).astype(np.float32)
    yp = g.standard_normal((T * k, H)).astype(np.float32)
    ys = g.standard_normal((T, H)).astype(np.float32)
    if act == "bf16":
        yp_d, ys_d = _bf16_dev(yp), _bf16_dev(ys)
        yp_v, ys_v = _dec(f32_to_bf16_bits(yp)), _dec(f32_to_bf16_bits(ys))
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        tol = 2 ** -8
    else:
        yp_d, ys_d, yp_v, ys_v = dev_f32(yp), dev_f32(ys), yp, ys
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        tol = 1e-6
    L.moe_combine(cfg, yp_d, ys_d, dev_i32(inv), dev_f32(w), y)
    torch.cuda.synchronize()
    ref = oracle.combine(yp_v, ys_v, inv, w)
    got = host(y)
    # elementwise as well: a dropped slot changes single elements by a whole term
    scale = np.abs(ref).max()
    assert np.abs(got - ref).max() < tol * scale
    assert rel_inf(got, ref) < tol


# ---------------------------------------------------------------- expert GEMMs on given routing
FFN_CASES = [
    # (T, H, E, G, M, k, S, I) -- several tiles, ragged row tails, shared experts
    (300, 256, 8, 2, 2, 2, 1, 256),
    (517, 320, 16, 4, 2, 4, 2, 128),
    (64, 512, 4, 4, 4, 4, 0, 384),
    (1, 256, 8, 2, 1, 2, 1, 128),
    (1000, 1024, 64, 8, 3, 6, 2, 256),
    (300, 576, 32, 4, 2, 16, 1, 128),   # combine rows of 72 chunks with k = 16 slots
]


@pytest.mark.parametrize("T,H,E,G,M,k,S,I", FFN_CASES)
def test_expert_ffn_bf16(T, H, E, G, M, k, S, I):
    say(f"ffn bf16 T={T} H={H} E={E} k={k} S={S} I={I}")
    c = MID.with_(T=T, H=H, E=E, G=G, M=M, k=k, S=S, I=I, sigma=0.05, group_topr=min(2, E // G))
    wts = make_weights(c)
    xb = make_x(c)
    s32 = oracle.affinity(_dec(xb), _dec(wts.w_router), wts.logit_offset)
    layer = MoeLayerGPU(c, wts)
    x = to_device(xb)
    bias = dev_f32(wts.bias0)
    layer.scores.copy_(dev_f32(s32))
    y = layer.forward(x, bias, scores_in=True)
    torch.cuda.synchronize()
    ref = oracle.forward_from_routing(c, xb, wts, wts.bias0, s32, *oracle.route(
        s32, wts.bias0, c.G, c.M, c.k, c.group_topr, c.route_scale))
    assert (host(layer.topk_idx) == ref["idx"]).all()
    assert (host(layer.offsets) == ref["offsets"]).all()
    e_p = rel_inf(host(layer.y_perm), ref["y_perm"])
    e_y = rel_inf(host(y), ref["y"])
    say(f"  y_perm err {e_p:.2e}  y err {e_y:.2e}")
    assert e_p < 2e-2 and e_y < 2e-2
    if S:
        assert rel_inf(host(layer.y_shared), ref["y_shared"]) < 2e-2


# ---------------------------------------------------------------- whole layer, multi-step
def _check_route(c, s_gpu, bias, idx_gpu):
    """Teacher-forced routing check: the oracle routes the GPU's own fp32 scores with
    the GPU's current bias; indices must agree bit for bit."""
    idx_o, w_o = oracle.route(s_gpu, bias, c.G, c.M, c.k, c.group_topr, c.route_scale)
    assert (idx_gpu == idx_o).all()
    return w_o


def _check_full_route(c, s_ora, bias, idx_gpu):
    """Own-scores routing check: mismatches only at near-ties of the oracle."""
    idx_o, _ = oracle.route(s_ora, bias, c.G, c.M, c.k, c.group_topr, c.route_scale)
    gk, gm = oracle.route_diagnostics(s_ora, bias, c.G, c.M, c.k, c.group_topr)
    # the selected set may differ only at a near-tie (slot order within a set may differ
    # wherever two selected scores are within rounding of each other)
    bad = (np.sort(idx_o, axis=1) != np.sort(idx_gpu, axis=1)).any(axis=1)
    assert ((gk[bad] < GAP) | (gm[bad] < GAP)).all()
    return int(bad.sum())


def test_layer_tiny_fp32_ten_steps():
    c = TINY
    wts = make_weights(c)
    layer = MoeLayerGPU(c, wts)
    bias_h = wts.bias0.copy()
    bias = dev_f32(bias_h)
    for step in range(c.steps):
        say(f"tiny fp32 step {step}")
        xh = make_x(c, step)
        y = layer.forward(to_device(xh), bias, gamma=c.gamma)
        torch.cuda.synchronize()
        s_gpu = host(layer.scores)
        s_ora = oracle.affinity(xh, wts.w_router, wts.logit_offset)
        assert np.abs(s_gpu - s_ora).max() < 1e-6
        idx = host(layer.topk_idx)
        w_o = _check_route(c, s_gpu, bias_h, idx)
        _check_full_route(c, s_ora, bias_h, idx)
        np.testing.assert_allclose(host(layer.topk_w), w_o, rtol=2e-6, atol=1e-7)
        sel = np.take_along_axis(s_ora.astype(np.float64), idx.astype(np.int64), 1)
        w_tf = c.route_scale * sel / sel.sum(1, keepdims=True)    # oracle gates on the GPU's selection
        ref = oracle.forward_from_routing(c, xh, wts, bias_h, s_ora, idx, w_tf)
        assert (host(layer.counts) == ref["counts"]).all()
        assert (host(layer.perm) == ref["perm"]).all()
        assert rel_inf(host(y), ref["y"]) < 1e-4
        bias_next = oracle.update_bias(bias_h, ref["counts"], c.T, c.k, c.gamma)
        assert (host(bias).view(np.uint32) == bias_next.view(np.uint32)).all()
        bias_h = bias_next


def test_layer_mid_bf16_balance_loop():
    """The mid configuration (T=4096, 64 experts, Zipf-skewed logits): 50 batches of
    routing + bias update, teacher-forced bit-exact per step; the layer output of
    the first and last step on a token sample."""
    c = MID
    wts = make_weights(c)
    layer = MoeLayerGPU(c, wts)
    bias_h = wts.bias0.copy()
    bias = dev_f32(bias_h)
    wr = _dec(wts.w_router)
    ratios = []
    for step in range(c.steps):
        xh = make_x(c, step)
        say(f"mid bf16 step {step}")
        y = layer.forward(to_device(xh), bias, gamma=c.gamma)
        torch.cuda.synchronize()
        s_gpu = host(layer.scores)
        idx = host(layer.topk_idx)
        _check_route(c, s_gpu, bias_h, idx)
        counts = host(layer.counts)
        assert (counts == np.bincount(idx.ravel(), minlength=c.E)).all()
        ratios.append(counts.max() / (c.T * c.k / c.E))
        if step in (0, c.steps - 1):
            s_ora = oracle.affinity(_dec(xh), wr, wts.logit_offset)
            assert np.abs(s_gpu - s_ora).max() < 1e-4
            nbad = _check_full_route(c, s_ora, bias_h, idx)
            say(f"  near-tie index flips: {nbad}")
            rows = rng(step, 5).choice(c.T, 128, replace=False)
            sel = np.take_along_axis(s_ora[rows].astype(np.float64), idx[rows].astype(np.int64), 1)
            w_rows = c.route_scale * sel / sel.sum(1, keepdims=True)
            ref = oracle.sampled_forward(c, xh[rows], idx[rows], w_rows, wts)
            err = rel_inf(host(y)[rows], ref)
            say(f"  sampled y err {err:.2e}")
            assert err < 2e-2
        bias_next = oracle.update_bias(bias_h, counts, c.T, c.k, c.gamma)
        assert (host(bias).view(np.uint32) == bias_next.view(np.uint32)).all()
        bias_h = bias_next
    say(f"  max/mean load first {ratios[0]:.2f} last {ratios[-1]:.2f}")
    assert ratios[-1] < ratios[0]


def test_layer_determinism_and_routing_invariants():
    """Two runs of the same batch give bitwise-equal routing, dispatch, bias and
    layer output; on the GPU's own outputs every token uses at most M groups and
    its gates sum to the gate scale (to k ulps), and gates recomputed from the
    GPU's fp32 affinities equal the GPU's gates (the bias never enters them)."""
    c = MID.with_(T=2048)
    wts = make_weights(c)
    layer = MoeLayerGPU(c, wts)
    xh = make_x(c, 0)
    outs = []
    for run in range(2):
        say(f"mid bf16 determinism run {run}")
        bias = dev_f32(wts.bias0)
        y = layer.forward(to_device(xh), bias, gamma=c.gamma)
        torch.cuda.synchronize()
        outs.append({n: host(getattr(layer, n)).copy() for n in ("topk_idx", "topk_w", "counts", "offsets",
                                                                   "perm", "inv", "scores")})
        outs[-1]["y"] = host(y).copy()
        outs[-1]["bias"] = host(bias).copy()
    for n in outs[0]:
        a, b = outs[0][n], outs[1][n]
        assert a.dtype == b.dtype and (a.view(np.uint8) == b.view(np.uint8)).all(), n
    idx, w, s = outs[0]["topk_idx"], outs[0]["topk_w"], outs[0]["scores"]
    groups = idx // (c.E // c.G)
    assert max(len(set(r)) for r in groups) <= c.M
    ulp = np.spacing(np.float32(c.route_scale))
    assert np.abs(w.astype(np.float64).sum(1) - c.route_scale).max() <= c.k * ulp
    sel = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), 1)
    np.testing.assert_allclose(w, c.route_scale * sel / sel.sum(1, keepdims=True), rtol=2e-6, atol=0)


@pytest.mark.parametrize("T,E", [(1, 256), (128, 256), (300, 200), (1000, 256), (2048, 256), (2049, 256),
                                 (8192, 256), (16384, 256), (16384, 192), (12345, 64), (16384, 64), (32768, 64),
                                 (65613, 64)])
def test_router_gemm_tile_heights(T, E):
    """The router's kernel and tile follow the batch on a 256-CU chip: the split-K kernel
    with 16 x 16 tiles (T = 1, 128; T = 300 with ragged token and expert tiles) and
    32 x 32 tiles (T = 1000, 2048); then, while no larger tile fills the chip, the fused
    kernel (router GEMM with the top-k in its epilogue) with 64-token tiles of all experts
    (E = 256: T = 2049 with one token in the last tile, 8192; E = 64: T = 12345, 16384);
    then the two-kernel path with 128 x 128 tiles (T = 16384, E = 256, and E = 192 with
    a ragged second column tile), 128 x 256 (T = 32768, E = 64) and 256 x 256 (T = 65613,
    ragged last row tile).  Affinities against the fp64 oracle, routing teacher-forced bit
    for bit; the same call without the affinities and the top-k alone on the written
    affinities give the same indices and gates bit for bit."""
    from biased_top_routing_amd import _lib as L
    c = MID.with_(T=T, H=256, E=E, I=128, S=1)
    w = make_weights(c)
    xh = make_x(c)
    say(f"router T={T} E={E}")
    cfg = L.cfg_from(c)
    x, wr, off, b = to_device(xh), to_device(w.w_router), to_device(w.logit_offset), dev_f32(w.bias0)
    s = torch.empty((T, c.E), dtype=torch.float32, device="cuda")
    outs = []
    for mode in ("scores", "no scores", "scores in"):
        idx = torch.full((T, c.k), -1, dtype=torch.int32, device="cuda")
        wt = torch.full((T, c.k), -1.0, dtype=torch.float32, device="cuda")
        if mode == "scores":
            L.moe_route(cfg, x, wr, off, b, s, 0, idx, wt)
        elif mode == "no scores":
            ws = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_ROUTE), dtype=torch.uint8, device="cuda")
            L.moe_route(cfg, x, wr, off, b, None, 0, idx, wt, ws)
        else:
            L.moe_route(cfg, None, None, None, b, s, L.MOE_SCORES_IN, idx, wt)
        torch.cuda.synchronize()
        outs.append((host(idx), host(wt)))
    s_gpu = host(s)
    s_ora = oracle.affinity(oracle.decode_act(xh).astype(np.float64), oracle.decode_act(w.w_router).astype(np.float64),
                            w.logit_offset)
    assert np.abs(s_gpu - s_ora).max() < 1e-5
    idx_o, w_o = oracle.route(s_gpu, w.bias0, c.G, c.M, c.k, c.group_topr, c.route_scale)
    assert (outs[0][0] == idx_o).all()
    np.testing.assert_allclose(outs[0][1], w_o, rtol=2e-6, atol=1e-7)
    for idx_m, w_m in outs[1:]:
        assert (idx_m == outs[0][0]).all()
        assert (w_m.view(np.uint32) == outs[0][1].view(np.uint32)).all()


@pytest.mark.parametrize("T", [1, 255, 256, 1000])
def test_router_fp32_with_and_without_scores(T):
    """The fp32 path (one thread per logit, then the top-k): the call without the
    affinities stages them in the workspace and gives the indices and gates of the call
    that writes them, bit for bit; those affinities match the fp64 oracle and the routing
    is the oracle's on them."""
    c = TINY.with_(T=T)
    w = make_weights(c)
    xh = make_x(c)
    say(f"fp32 router T={T}")
    cfg = L.cfg_from(c)
    x, wr, off, b = to_device(xh), to_device(w.w_router), to_device(w.logit_offset), dev_f32(w.bias0)
    s = torch.full((T, c.E), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((L.moe_workspace_bytes(cfg, L.MOE_WS_ROUTE),), 0xFF, dtype=torch.uint8, device="cuda")
    outs = []
    for scores in (s, None):
        idx = torch.full((T, c.k), -1, dtype=torch.int32, device="cuda")
        wt = torch.full((T, c.k), -1.0, dtype=torch.float32, device="cuda")
        L.moe_route(cfg, x, wr, off, b, scores, 0, idx, wt, None if scores is not None else ws)
        torch.cuda.synchronize()
        outs.append((host(idx), host(wt)))
    s_gpu = host(s)
    assert np.abs(s_gpu - oracle.affinity(xh, w.w_router, w.logit_offset)).max() < 1e-6
    idx_o, w_o = oracle.route(s_gpu, w.bias0, c.G, c.M, c.k, c.group_topr, c.route_scale)
    assert (outs[0][0] == idx_o).all()
    np.testing.assert_allclose(outs[0][1], w_o, rtol=2e-6, atol=1e-7)
    assert (outs[1][0] == outs[0][0]).all()
    assert (outs[1][1].view(np.uint32) == outs[0][1].view(np.uint32)).all()


# ---------------------------------------------------------------- gate/up row tiling boundaries
SEG_SIZES = [1, 96, 128, 129, 160, 161, 192, 256, 257, 320, 321, 384, 512, 513, 576, 640, 641, 700, 768, 769]


def test_expert_segments_at_row_tile_boundaries():
    """Expert segments at every boundary of the row tiling (gate/up: 320-row tiles, or 256-row
    tiles where that takes no more of them, wavefront bands of 160 / 128 rows; down: 256-row
    tiles, 64-row bands), routed from given scores (top-1 of 20 experts, one group): every
    segment's y_perm against the fp64 oracle, and the gather and keep-g,u entry points bit
    for bit against the row-copy one."""
    E, T = len(SEG_SIZES), sum(SEG_SIZES)
    c = MID.with_(T=T, H=256, E=E, G=1, M=1, k=1, S=1, I=256, group_topr=1, sigma=0.05)
    w = make_weights(c)
    xb = make_x(c)
    target = rng(7, 1).permutation(np.repeat(np.arange(E), SEG_SIZES))
    s32 = np.full((T, E), 0.25, np.float32)
    s32[np.arange(T), target] = 0.75
    say(f"segments at tile boundaries: T={T}, E={E}")
    outs = {}
    for mode in ("copy", "gather", "save"):
        layer = MoeLayerGPU(c, w, gather=mode == "gather", save_gu=mode == "save")
        layer.scores.copy_(dev_f32(s32))
        layer.forward(to_device(xb), dev_f32(w.bias0), scores_in=True)
        torch.cuda.synchronize()
        outs[mode] = (host(layer.y_perm), host(layer.y), host(layer.offsets))
    ref = oracle.forward_from_routing(c, xb, w, w.bias0, s32, *oracle.route(
        s32, w.bias0, c.G, c.M, c.k, c.group_topr, c.route_scale))
    yp, y, offs = outs["copy"]
    assert (offs == np.concatenate([[0], np.cumsum(SEG_SIZES)])).all()
    for e in range(E):
        lo, hi = offs[e], offs[e + 1]
        err = rel_inf(yp[lo:hi], ref["y_perm"][lo:hi])
        assert err < 2e-2, (e, SEG_SIZES[e], err)
    assert rel_inf(y, ref["y"]) < 2e-2
    for mode in ("gather", "save"):
        assert (outs[mode][0].view(np.uint32) == yp.view(np.uint32)).all(), f"{mode}: y_perm bits differ"
        assert (outs[mode][1].view(np.uint32) == y.view(np.uint32)).all(), f"{mode}: y bits differ"


def test_layer_resume_from_saved_bias(tmp_path):
    """The bias is the layer's only state across batches.  Ten batches in one run equal
    five batches, the bias written to a file and read back into a freshly built layer,
    then five more batches: the layer outputs of batches 5..9 and the final bias are
    identical bit for bit (tiny fp32 workload, fresh x per batch)."""
    c = TINY
    wts = make_weights(c)
    xs = [make_x(c, step) for step in range(10)]

    def run(layer, bias, steps):
        ys = []
        for step in steps:
            say(f"resume test batch {step}")
            ys.append(host(layer.forward(to_device(xs[step]), bias, gamma=c.gamma)).copy())
        torch.cuda.synchronize()
        return ys

    bias_a = dev_f32(wts.bias0)
    ys_a = run(MoeLayerGPU(c, wts), bias_a, range(10))
    bias_b = dev_f32(wts.bias0)
    run(MoeLayerGPU(c, wts), bias_b, range(5))
    path = tmp_path / "bias.npy"
    np.save(path, host(bias_b))
    bias_c = dev_f32(np.load(path))
    ys_c = run(MoeLayerGPU(c, wts), bias_c, range(5, 10))
    for a, b in zip(ys_a[5:], ys_c):
        assert (a.view(np.uint32) == b.view(np.uint32)).all()
    assert (host(bias_a).view(np.uint32) == host(bias_c).view(np.uint32)).all()
