"""GPU parity of the fine-grained FP8 path (E4M3 codes, one fp32 scale per 1 x 128
activation tile and per 128 x 128 weight block).

Quantisation is integer-valued work decided in fp32 on both sides (scale
fl32(amax/448), value fl32(v/sc), nearest-even E4M3), so codes and scales are
compared bit for bit: the whole E4M3 range on a sweep of every bf16 value, random
rows and weight blocks, and the quantising dispatch.  The FP8 expert GEMMs are
compared with the quantisation-emulating oracle (exact code products per 128-K
chunk, scaled, accumulated in fp64) at the normwise 6e-2 bound; the GPU's h is
computed in fp32 before its own quantisation, so an h code can sit one step away
from the oracle's where h falls near a rounding boundary."""
import numpy as np
import pytest
import torch

import oracle
from biased_top_routing_amd import _lib as L
from biased_top_routing_amd.runner import MoeLayerGPU, to_device
from gpu_util import dev_f32, dev_i32, host, rel_inf, sample_tokens, say
from workloads import MID, V3_FP8
from workloads.inputs import f32_to_bf16_bits, make_weights, make_x, rng

pytestmark = pytest.mark.gpu

TOL = 6e-2
GAP = 1e-5


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _quant_rows_gpu(bits):
    R, K = bits.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty((R, K // 128), dtype=torch.float32, device="cuda")
    L.moe_quantize_fp8(_bf16_dev(bits), 1, R, K, 1, codes, sc)
    torch.cuda.synchronize()
    return host(codes), host(sc)


# ---------------------------------------------------------------- quantisation, bit-exact
def test_e4m3_encode_sweep_every_bf16_value():
    """Every finite bf16 value of magnitude <= 448 (including every E4M3 midpoint and
    its bf16 neighbours), in tiles whose first element is 448 so that the scale is 1."""
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = oracle.decode_act(u)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    vals = u[keep]
    n_tiles = -(-len(vals) // 127)
    pad = np.full(n_tiles * 127 - len(vals), f32_to_bf16_bits(np.float32(1.0)), np.uint16)
    body = np.concatenate([vals, pad]).reshape(n_tiles, 127)
    first = np.full((n_tiles, 1), f32_to_bf16_bits(np.float32(448.0)), np.uint16)
    tiles = np.concatenate([first, body], axis=1)
    say(f"e4m3 sweep: {len(vals)} bf16 values in {n_tiles} tiles")
    codes, sc = _quant_rows_gpu(tiles)
    assert (sc == 1.0).all()
    ref = oracle.e4m3_encode(oracle.decode_act(tiles))
    assert (codes == ref).all()


@pytest.mark.parametrize("R,K", [(37, 128), (300, 896), (5, 7168)])
def test_quantize_rows_exact(R, K):
    g = rng(21, R, K)
    x = g.standard_normal((R, K)).astype(np.float32) * np.exp(g.uniform(-12, 6, (R, 1))).astype(np.float32)
    x[0, :128] = 0.0                                  # all-zero tile: scale 1
    x[1 % R, 5] = 1e4                                 # one outlier widens only its own tile
    bits = f32_to_bf16_bits(x)
    say(f"quantize rows {R}x{K}")
    codes, sc = _quant_rows_gpu(bits)
    qr, sr = oracle.quantize_rows_1x128(oracle.decode_act(bits))
    assert (sc.view(np.uint32) == sr.view(np.uint32)).all()
    assert (codes == qr).all()


def test_quantize_blocks_exact():
    n, R, K = 3, 256, 384
    g = rng(22, n)
    w = (g.standard_normal((n, R, K)) * 0.006).astype(np.float32)
    w[1, :128, :128] = 0.0
    w[2, 200, 300] = 3.0
    bits = f32_to_bf16_bits(w)
    codes = torch.empty((n, R, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty((n, R // 128, K // 128), dtype=torch.float32, device="cuda")
    say("quantize 128x128 blocks")
    L.moe_quantize_fp8(_bf16_dev(bits), n, R, K, 128, codes, sc)
    torch.cuda.synchronize()
    for i in range(n):
        qb, sb = oracle.quantize_blocks_128x128(oracle.decode_act(bits[i]))
        assert (host(sc)[i].view(np.uint32) == sb.view(np.uint32)).all()
        assert (host(codes)[i] == qb).all()


def test_dispatch_fp8_exact():
    c = MID.with_(T=700, H=384, E=16, G=4, M=2, k=4, S=1, I=256, wgt="fp8_e4m3", group_topr=2)
    g = rng(23, 1)
    s = g.random((c.T, c.E)).astype(np.float32)
    idx, _ = oracle.route(s, np.zeros(c.E, np.float32), c.G, c.M, c.k, c.group_topr, c.route_scale)
    xb = make_x(c)
    cfg = L.cfg_from(c)
    P = c.T * c.k
    counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(c.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(P, dtype=torch.int32, device="cuda")
    inv = torch.empty((c.T, c.k), dtype=torch.int32, device="cuda")
    xq = torch.empty((P, c.H), dtype=torch.uint8, device="cuda")
    xs = torch.empty((P, c.H // 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_DISPATCH), dtype=torch.uint8, device="cuda")
    say("fp8 dispatch")
    L.moe_dispatch(cfg, dev_i32(idx), to_device(xb), counts, offsets, perm, inv, xq, xs, ws)
    torch.cuda.synchronize()
    _, off_o, perm_o, inv_o = oracle.dispatch(idx, c.E)
    assert (host(perm) == perm_o).all() and (host(inv) == inv_o).all()
    qr, sr = oracle.quantize_rows_1x128(oracle.decode_act(xb))
    assert (host(xq) == qr[perm_o // c.k]).all()
    assert (host(xs).view(np.uint32) == sr[perm_o // c.k].view(np.uint32)).all()


# ---------------------------------------------------------------- FP8 expert GEMMs on given routing
FFN8_CASES = [
    # (T, H, E, G, M, k, S, I): several tiles, ragged row tails, shared experts,
    # odd numbers of 128-column blocks, K up to the 64-chunk limit
    (300, 256, 8, 2, 2, 2, 1, 256),
    (517, 384, 16, 4, 2, 4, 2, 128),
    (64, 512, 4, 4, 4, 4, 0, 384),
    (1, 256, 8, 2, 1, 2, 1, 128),
    (1000, 1024, 64, 8, 3, 6, 2, 256),
    (200, 7168, 8, 2, 2, 2, 1, 256),
    (130, 8192, 4, 2, 1, 2, 1, 128),
    # K in whole groups of 4 chunks (activation scales loaded 4 chunks at a time) in both GEMMs:
    # one group (H = 512), the shared down GEMM over 2 experts' 8 chunks; 3 groups (H = 1536)
    (300, 512, 16, 4, 2, 4, 2, 512),
    (257, 1536, 8, 2, 2, 2, 1, 1024),
]


def _spread(bits, g, rows_per_block):
    """Multiply every rows_per_block x 128 block of a bf16 array by its own power of two
    in [2^-3, 2^3] (exact in bf16), so that tiles and blocks get very different scales
    and a scale applied to the wrong chunk, row or block shows up as a large error."""
    v = oracle.decode_act(bits)
    sh = v.shape
    R, K = sh[-2], sh[-1]
    b = v.reshape(-1, R // rows_per_block, rows_per_block, K // 128, 128)
    f = np.exp2(g.integers(-3, 4, (b.shape[0], b.shape[1], 1, b.shape[3], 1))).astype(np.float32)
    return f32_to_bf16_bits((b * f).reshape(sh))


# The FP8 MFMA of gfx950 does not sum a chunk's products exactly: on E4M3 codes with a
# wide exponent range its result is off by up to about 5.3e-4 of the chunk's largest
# product (measured on MI355X for 16x16x128 and 32x32x64, from a zero accumulator; the
# add into the accumulator is one fp32 rounding); codes of a narrow exponent range sum
# exactly.  It is the analogue of the limited FP8 accumulation precision the pages report
# for their hardware, and promoting each 128-element chunk into fp32 keeps it from
# growing with K.  The checks below allow EPS_MFMA times the chunk's largest |product|
# (or, where that is too slow to compute, the sum of |products|, an upper bound of it)
# per chunk, propagated through SwiGLU, the 1 x 128 quantisation of h and the down GEMM;
# everything else is fp32 rounding.
EPS_MFMA = 2.0 ** -10
F32_SLACK = 2.0 ** -21


def _mfma_bound(qa, sa, qw, sw, tight):
    """Sum over 128-K chunks of scale * (largest |product| of the chunk) when tight, else
    of scale * (sum of |products|), which is larger and much cheaper."""
    if not tight:
        return oracle.fp8_matmul(qa & 0x7F, sa, qw & 0x7F, sw)
    A = np.abs(oracle.e4m3_decode(qa))
    W = np.abs(oracle.e4m3_decode(qw))
    R, K = A.shape
    out = np.zeros((R, W.shape[0]))
    for c in range(K // 128):
        a, w = A[:, c * 128:(c + 1) * 128], W[:, c * 128:(c + 1) * 128]
        scale = np.asarray(sa, np.float64)[:, c:c + 1] * np.repeat(np.asarray(sw, np.float64)[:, c], 128)[None, :]
        for r0 in range(0, R, 32):
            out[r0:r0 + 32] += (a[r0:r0 + 32, None, :] * w[None, :, :]).max(axis=2) * scale[r0:r0 + 32]
    return out


def _gate_up_model(fe, qx, sx, tight=True):
    """Oracle h (fp64) of E4M3 rows and the bound on |h_gpu - h| the MFMA error allows."""
    I, kb = fe.I, fe.I // 128
    parts = []
    for rows, srows in ((slice(0, I), slice(0, kb)), (slice(I, 2 * I), slice(kb, 2 * kb))):
        q, sw = fe.qgu[rows], fe.sgu[srows]
        v = oracle.fp8_matmul(qx, sx, q, sw)
        parts.append((v, EPS_MFMA * _mfma_bound(qx, sx, q, sw, tight) + F32_SLACK * np.abs(v)))
    (g, dg), (u, du) = parts
    h = fe.hidden(qx, sx)
    silu = g / (1.0 + np.exp(-g))
    # |d silu / dg| <= 1.1 everywhere
    dh = 1.1 * dg * (np.abs(u) + du) + np.abs(silu) * du + F32_SLACK * np.abs(h)
    return h, dh


def _check_h(h64, dh, hq, hs):
    """GPU-quantised h (codes hq, tile scales hs) against the oracle's fp64 h and its
    allowed deviation dh: each tile scale is the amax/448 of some h within the bounds,
    and each code is the nearest E4M3 value of some h/scale within the bounds.
    Returns (fraction of codes equal to the oracle's own, largest scale deviation)."""
    n, I = h64.shape
    t, dt = h64.reshape(n, I // 128, 128), dh.reshape(n, I // 128, 128)
    amax = np.abs(t).max(axis=2)
    ref_sc = np.where(amax == 0, 1.0, amax / 448.0)
    sc_slack = dt.max(axis=2) / 448.0 + 2.0 ** -22 * ref_sc
    dev = float((np.abs(hs - ref_sc) / ref_sc).max()) if hs.size else 0.0
    assert (np.abs(hs - ref_sc) <= sc_slack).all(), dev
    u, su = t / hs[:, :, None], dt / hs[:, :, None]              # h and its slack in the GPU's scale units
    dq = oracle.e4m3_decode(hq.reshape(n, I // 128, 128))
    e = np.floor(np.log2(np.maximum(np.abs(u) + su, 2.0 ** -6)))
    half = 0.5 * np.exp2(e - 3)
    miss = np.abs(dq - np.clip(u, -448, 448)) - (half + su + 1e-12)
    if (miss > 0).any():
        bad = np.argsort(miss.ravel())[::-1][:6]
        for b in bad:
            say(f"    code off: u={u.ravel()[b]:.6g} dq={dq.ravel()[b]:.6g} half-step={half.ravel()[b]:.3g} "
                f"slack={su.ravel()[b]:.3g}")
        say(f"    {int((miss > 0).sum())} of {miss.size} codes outside the bound")
    assert (miss <= 0).all()
    q_ref, _ = oracle.quantize_rows_1x128(h64.astype(np.float32))
    same = float((q_ref == hq).mean())
    assert same > 0.95, same
    return same, dev


def _check_down(y_gpu, fdowns, tight=True):
    """y_gpu (bf16) against the oracle's down GEMM(s) of the GPU's own h: the MFMA bound
    plus one bf16 rounding, element by element.  fdowns: list of (expert, h codes, scales)."""
    yr = np.zeros(y_gpu.shape)
    ya = np.zeros(y_gpu.shape)
    for fe, q, sc in fdowns:
        yr += fe.down(q, sc)
        ya += _mfma_bound(q, sc, fe.qd, fe.sd, tight)
    bound = 2.0 ** -8 * np.abs(yr) + EPS_MFMA * ya * (1 + 2.0 ** -8) + F32_SLACK * np.abs(yr)
    assert (np.abs(y_gpu - yr) <= bound + 1e-30).all()


def _ws_part(layer, part, shape, dtype):
    off, nb = L.moe_ffn_workspace_part(layer.cfg, part)
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    assert n <= nb
    return host(layer.ws_ffn[off:off + n].view(dtype).view(*shape))


def _check_fp8_intermediates(c, layer, xq_rows_of, wts):
    """h of every routed segment and of the shared experts, and the down GEMM applied to
    the GPU's own h (bf16 output rounding only: 2^-8)."""
    P = c.T * c.k
    offsets = host(layer.offsets)
    hq = _ws_part(layer, L.MOE_WSP_H, (P, c.I), torch.uint8)
    hs = _ws_part(layer, L.MOE_WSP_H_SCALE, (P, c.I // 128), torch.float32)
    yp = host(layer.y_perm)
    worst, wdev = 1.0, 0.0
    for e in range(c.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        fe = oracle.layer._Fp8Expert(wts.w_gate_up[e], wts.w_down[e])
        qx, sx = xq_rows_of(slice(lo, hi))
        same, dev = _check_h(*_gate_up_model(fe, qx, sx), hq[lo:hi], hs[lo:hi])
        worst, wdev = min(worst, same), max(wdev, dev)
        _check_down(yp[lo:hi], [(fe, hq[lo:hi], hs[lo:hi])])
    if c.S:
        hq_s = _ws_part(layer, L.MOE_WSP_H_SHARED, (c.T, c.S * c.I), torch.uint8)
        hs_s = _ws_part(layer, L.MOE_WSP_H_SHARED_SCALE, (c.T, c.S * c.I // 128), torch.float32)
        qx, sx = xq_rows_of(None)
        downs = []
        for s in range(c.S):
            fs = oracle.layer._Fp8Expert(wts.ws_gate_up[s], wts.ws_down[s])
            cs, ct = slice(s * c.I, (s + 1) * c.I), slice(s * c.I // 128, (s + 1) * c.I // 128)
            same, dev = _check_h(*_gate_up_model(fs, qx, sx), hq_s[:, cs], hs_s[:, ct])
            worst, wdev = min(worst, same), max(wdev, dev)
            downs.append((fs, hq_s[:, cs], hs_s[:, ct]))
        _check_down(host(layer.y_shared), downs)
    return worst, wdev


@pytest.mark.parametrize("T,H,E,G,M,k,S,I", FFN8_CASES)
def test_expert_ffn_fp8(T, H, E, G, M, k, S, I):
    say(f"ffn fp8 T={T} H={H} E={E} k={k} S={S} I={I}")
    c = MID.with_(T=T, H=H, E=E, G=G, M=M, k=k, S=S, I=I, sigma=0.05, group_topr=min(2, E // G),
                  wgt="fp8_e4m3")
    wts = make_weights(c)
    g = rng(24, T, H, E, S, I)
    wts.w_gate_up, wts.w_down = _spread(wts.w_gate_up, g, 128), _spread(wts.w_down, g, 128)
    if S:
        wts.ws_gate_up, wts.ws_down = _spread(wts.ws_gate_up, g, 128), _spread(wts.ws_down, g, 128)
    xb = _spread(make_x(c), g, 1)
    s32 = oracle.affinity(oracle.decode_act(xb).astype(np.float64),
                          oracle.decode_act(wts.w_router).astype(np.float64), wts.logit_offset)
    layer = MoeLayerGPU(c, wts)
    bias = dev_f32(wts.bias0)
    layer.scores.copy_(dev_f32(s32))
    y = layer.forward(to_device(xb), bias, scores_in=True)
    torch.cuda.synchronize()
    idx, w = oracle.route(s32, wts.bias0, c.G, c.M, c.k, c.group_topr, c.route_scale)
    ref = oracle.forward_from_routing(c, xb, wts, wts.bias0, s32, idx, w)
    assert (host(layer.topk_idx) == ref["idx"]).all()
    qx_all, sx_all = oracle.quantize_rows_1x128(oracle.decode_act(xb))
    perm_tok = ref["perm"] // c.k
    same, dev = _check_fp8_intermediates(
        c, layer, lambda rows: (qx_all, sx_all) if rows is None else (qx_all[perm_tok[rows]], sx_all[perm_tok[rows]]),
        wts)
    e_p = rel_inf(host(layer.y_perm), ref["y_perm"])
    e_y = rel_inf(host(y), ref["y"])
    e_s = rel_inf(host(layer.y_shared), ref["y_shared"]) if S else 0.0
    say(f"  h codes equal to the oracle's: {same:.5f} (scale dev {dev:.1e}); y_perm err {e_p:.2e}  "
        f"y_shared err {e_s:.2e}  "
        f"y err {e_y:.2e}")
    assert e_p < TOL and e_y < TOL and e_s < TOL


# ---------------------------------------------------------------- V3-like FP8 layer at full size
@pytest.fixture(scope="module")
def v3_fp8():
    say("v3 fp8: generating weights (22.5 GB bf16)")
    w = make_weights(V3_FP8)
    say("v3 fp8: uploading and quantising on the GPU")
    layer = MoeLayerGPU(V3_FP8, w)
    torch.cuda.synchronize()
    return w, layer


def test_v3_fp8_full_size(v3_fp8):
    """T=32768 tokens, 256 experts, Zipf-skewed logits: routing, dispatch and the
    bias update over the whole batch (teacher-forced, bit-exact), x_perm codes on
    sampled rows (bit-exact), one expert's whole segment, the shared expert on
    sampled tokens and the layer output of sampled tokens (6e-2)."""
    w, layer = v3_fp8
    c = V3_FP8
    xh = make_x(c, 0)
    bias_h = w.bias0.copy()
    bias = dev_f32(bias_h)
    say(f"v3 fp8 forward T={c.T}")
    y = layer.forward(to_device(xh), bias, gamma=c.gamma)
    torch.cuda.synchronize()
    y = host(y)
    s_gpu = host(layer.scores)
    idx = host(layer.topk_idx)
    idx_o, w_o = oracle.route(s_gpu, bias_h, c.G, c.M, c.k, c.group_topr, c.route_scale)
    assert (idx == idx_o).all()
    np.testing.assert_allclose(host(layer.topk_w), w_o, rtol=2e-6, atol=1e-7)
    counts, offsets, perm, inv = oracle.dispatch(idx, c.E)
    assert (host(layer.counts) == counts).all() and (host(layer.offsets) == offsets).all()
    assert (host(layer.perm) == perm).all() and (host(layer.inv) == inv).all()
    exp_b = oracle.update_bias(bias_h, counts, c.T, c.k, c.gamma)
    assert (host(bias).view(np.uint32) == exp_b.view(np.uint32)).all()
    say(f"  max/mean load {counts.max() / (c.T * c.k / c.E):.2f}")
    # own scores: index flips only at near-ties
    s_ora = oracle.affinity(oracle.decode_act(xh).astype(np.float64),
                            oracle.decode_act(w.w_router).astype(np.float64), w.logit_offset)
    assert np.abs(s_gpu - s_ora).max() < 1e-4
    ref_idx, _ = oracle.route(s_ora, bias_h, c.G, c.M, c.k, c.group_topr, c.route_scale)
    gk, gm = oracle.route_diagnostics(s_ora, bias_h, c.G, c.M, c.k, c.group_topr)
    bad = (np.sort(ref_idx, axis=1) != np.sort(idx, axis=1)).any(axis=1)
    assert ((gk[bad] < GAP) | (gm[bad] < GAP)).all()
    say(f"  near-tie index flips: {int(bad.sum())} of {c.T}")
    # quantising dispatch on sampled permuted rows
    prow = np.sort(rng(31, 1).choice(c.T * c.k, 256, replace=False))
    qr, sr = oracle.quantize_rows_1x128(oracle.decode_act(xh[perm[prow] // c.k]))
    assert (host(layer.x_perm[torch.from_numpy(prow).cuda()]) == qr).all()
    assert (host(layer.x_perm_scale[torch.from_numpy(prow).cuda()]).view(np.uint32) == sr.view(np.uint32)).all()
    # one expert's whole segment: the median load among experts with at least one row
    nz = np.flatnonzero(counts)
    e = int(nz[np.argsort(counts[nz])[len(nz) // 2]])
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    say(f"  expert {e}: {hi - lo} rows")
    fe = oracle.layer._Fp8Expert(w.w_gate_up[e], w.w_down[e])
    qx, sx = oracle.quantize_rows_1x128(oracle.decode_act(xh[perm[lo:hi] // c.k]))
    P = c.T * c.k
    hq = _ws_part(layer, L.MOE_WSP_H, (P, c.I), torch.uint8)[lo:hi]
    hs = _ws_part(layer, L.MOE_WSP_H_SCALE, (P, c.I // 128), torch.float32)[lo:hi]
    same, dev = _check_h(*_gate_up_model(fe, qx, sx, tight=False), hq, hs)
    ysg = host(layer.y_perm[lo:hi])
    _check_down(ysg, [(fe, hq, hs)], tight=False)
    err = rel_inf(ysg, fe(qx, sx))
    say(f"  h codes equal to the oracle's: {same:.5f} (scale dev {dev:.1e}); y_perm segment err {err:.2e}")
    assert err < TOL
    # shared expert and the layer output on 256 sampled tokens (the last 16 of the batch and
    # tokens of the largest, Zipf-hot, expert segment among them), teacher-forced on the
    # GPU's selection; the skewed routing keeps the experts they touch to a few dozen
    rows = sample_tokens(c.T, idx, 256, 32)
    cache = {e: (lambda rq, fe=fe: fe(*rq))}
    fs = oracle.layer._Fp8Expert(w.ws_gate_up[0], w.ws_down[0])
    cache[("shared", 0)] = lambda rq: fs(*rq)
    ref_s = fs(*oracle.quantize_rows_1x128(oracle.decode_act(xh[rows])))
    err = rel_inf(host(layer.y_shared)[rows], ref_s)
    say(f"  y_shared err on {len(rows)} sampled tokens {err:.2e}")
    assert err < TOL
    sel = np.take_along_axis(s_ora[rows].astype(np.float64), idx[rows].astype(np.int64), 1)
    w_rows = c.route_scale * sel / sel.sum(1, keepdims=True)
    say(f"  oracle layer output of {len(rows)} tokens over {len(np.unique(idx[rows]))} experts")
    ref_y = oracle.sampled_forward(c, xh[rows], idx[rows], w_rows, w, experts_cache=cache)
    err = rel_inf(y[rows], ref_y)
    say(f"  sampled y err {err:.2e}")
    assert err < TOL


def test_v3_fp8_hundred_balance_steps(v3_fp8):
    """The FP8 workload's 100 batches of routing + bias update (gamma = 1e-3, Zipf 1.5
    preference), each batch a fresh x from the shared generator (a prefix of T = 8192 of
    the full batch: the oracle routes every step's 8192 x 256 affinities in about a
    quarter of a second, where the full 32768 tokens would take about 1.5 s per step).
    Every step is checked teacher-forced and bit for bit: the oracle routes the GPU's
    fp32 affinities with the bias the GPU holds, and the indices, the per-expert loads
    and the updated bias must be identical; the gates within 2e-6."""
    w, layer = v3_fp8
    c = V3_FP8.with_(T=8192)
    layer.alloc(c.T)
    bias_h = w.bias0.copy()
    bias = dev_f32(bias_h)
    mean = c.T * c.k / c.E
    ratios = []
    for step in range(V3_FP8.steps):
        say(f"v3 fp8 balance step {step} T={c.T}")
        layer.forward(to_device(make_x(c, step, T=c.T)), bias, gamma=c.gamma)
        torch.cuda.synchronize()
        s_gpu = host(layer.scores)
        idx = host(layer.topk_idx)
        idx_o, w_o = oracle.route(s_gpu, bias_h, c.G, c.M, c.k, c.group_topr, c.route_scale)
        assert (idx == idx_o).all(), step
        np.testing.assert_allclose(host(layer.topk_w), w_o, rtol=2e-6, atol=1e-7)
        counts = host(layer.counts)
        assert (counts == np.bincount(idx.ravel(), minlength=c.E)).all(), step
        bias_next = oracle.update_bias(bias_h, counts, c.T, c.k, c.gamma)
        assert (host(bias).view(np.uint32) == bias_next.view(np.uint32)).all(), step
        bias_h = bias_next
        ratios.append(counts.max() / mean)
    say(f"  max/mean load step 1 {ratios[0]:.2f}, step 100 {ratios[-1]:.2f}")
    # the bias of the hottest expert fell by gamma every step (it is overloaded throughout)
    hot = int(np.argmax(counts))
    assert bias_h[hot] < w.bias0[hot] - 0.09
