"""GPU parity, bit-exact part: routing on given fp32 scores, dispatch, bias update.

Every call goes through the C ABI (libmoe.so); the expected values come from
the CPU oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
from biased_top_routing_amd import _lib as L
from gpu_util import dev_f32, dev_i32, host, say
from workloads.inputs import f32_to_bf16_bits, make_scores, rng

pytestmark = pytest.mark.gpu


def _route_gpu(scores, bias, E, G, M, k, r, scale):
    T = scores.shape[0]
    cfg = L.make_cfg(T, 128, E, G, M, k, 0, 128, r, scale, "bf16", "bf16")
    s = dev_f32(scores)
    b = dev_f32(bias)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    L.moe_route(cfg, None, None, None, b, s, L.MOE_SCORES_IN, idx, w)
    torch.cuda.synchronize()
    return host(idx), host(w)


ROUTE_CASES = [
    # (E, G, M, k, r, T, kind)
    (16, 4, 2, 4, 2, 257, "uniform"),
    (64, 8, 3, 6, 2, 1000, "uniform"),
    (256, 8, 4, 8, 2, 2049, "uniform"),
    (256, 8, 4, 8, 2, 700, "ties"),
    (256, 8, 4, 8, 1, 700, "ties"),
    (64, 8, 3, 6, 2, 600, "zeros"),
    (16, 4, 2, 4, 2, 300, "ties"),
    (512, 64, 8, 16, 3, 300, "uniform"),
    (96, 12, 5, 7, 4, 300, "ties"),
    (8, 1, 1, 8, 2, 100, "uniform"),
    (32, 32, 32, 32, 1, 100, "ties"),
    # the 16-lane form: one, two, four and eight lanes per group, top-r up to 4
    (128, 16, 4, 8, 3, 777, "uniform"),
    (256, 8, 4, 8, 4, 513, "ties"),
    (256, 4, 2, 8, 1, 400, "uniform"),
    (32, 2, 1, 4, 2, 333, "ties"),
    (256, 16, 4, 16, 2, 300, "zeros"),
    (64, 8, 3, 6, 2, 1, "uniform"),
]


@pytest.mark.parametrize("E,G,M,k,r,T,kind", ROUTE_CASES)
def test_route_scores_in_bit_exact(E, G, M, k, r, T, kind):
    say(f"route scores-in E={E} G={G} M={M} k={k} r={r} T={T} {kind}")
    s = make_scores(E * 7 + T, T, E, kind)
    b = rng(E, T, 1).uniform(-0.05, 0.05, E).astype(np.float32)
    if kind == "ties":
        b = (np.round(b * 8) / 8).astype(np.float32)
    idx_g, w_g = _route_gpu(s, b, E, G, M, k, r, 2.5)
    idx_o, w_o = oracle.route(s, b, G, M, k, r, 2.5)
    assert (idx_g == idx_o).all()
    np.testing.assert_allclose(w_g, w_o, rtol=2e-6, atol=1e-7)


def test_route_empty_batch():
    say("route T=0")
    cfg = L.make_cfg(0, 128, 16, 4, 2, 4, 0, 128, 2, 1.0, "bf16", "bf16")
    t = torch.empty(1, device="cuda")
    L.moe_route(cfg, None, None, None, t, t, L.MOE_SCORES_IN, t, t)
    torch.cuda.synchronize()


def _idx_random(seed, T, E, k, skew=None):
    g = rng(seed, 3)
    if skew == "one":      # every token picks experts 0..k-1
        return np.tile(np.arange(k, dtype=np.int32), (T, 1))
    keys = g.random((T, E))
    if skew == "zipf":
        keys = keys ** (1.0 / (np.arange(1, E + 1) ** -1.2))[None, :]
    return np.argsort(-keys, axis=1)[:, :k].astype(np.int32)


DISPATCH_CASES = [
    # (T, E, k, H, skew)
    (3000, 64, 6, 256, None),
    (100, 16, 4, 128, None),
    (16384, 256, 8, 64, None),
    (2000, 256, 8, 128, "zipf"),
    (777, 32, 3, 64, "one"),
    (130, 1, 1, 64, None),
]


@pytest.mark.parametrize("T,E,k,H,skew", DISPATCH_CASES)
def test_dispatch_bit_exact(T, E, k, H, skew):
    say(f"dispatch T={T} E={E} k={k} H={H} skew={skew}")
    G = 1
    cfg = L.make_cfg(T, H, E, G, 1, k, 0, 128, 1, 1.0, "bf16", "bf16")
    idx = _idx_random(T + E, T, E, k, skew)
    xb = f32_to_bf16_bits(rng(T, 4).standard_normal((T, H)).astype(np.float32))
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    P = T * k
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((P,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    xp = torch.empty((P, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_DISPATCH), dtype=torch.uint8, device="cuda")
    L.moe_dispatch(cfg, dev_i32(idx), x, counts, offsets, perm, inv, xp, None, ws)
    torch.cuda.synchronize()
    c_o, o_o, p_o, i_o = oracle.dispatch(idx, E)
    assert (host(counts) == c_o).all()
    assert (host(offsets) == o_o).all()
    assert (host(perm) == p_o).all()
    assert (host(inv) == i_o).all()
    xp_h = xp.view(torch.int16).cpu().numpy().view(np.uint16)
    assert (xp_h == oracle.permute_rows(xb, p_o, k)).all()
    # deterministic: a second run gives the same bits
    perm2 = torch.empty_like(perm)
    L.moe_dispatch(cfg, dev_i32(idx), x, counts, offsets, perm2, inv, xp, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(perm, perm2)


def test_dispatch_empty_batch_zeroes_counts():
    say("dispatch T=0")
    E = 16
    cfg = L.make_cfg(0, 64, E, 4, 2, 4, 0, 128, 2, 1.0, "bf16", "bf16")
    counts = torch.full((E,), 5, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), 5, dtype=torch.int32, device="cuda")
    t = torch.empty(16, dtype=torch.int32, device="cuda")
    ws = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_DISPATCH), dtype=torch.uint8, device="cuda")
    L.moe_dispatch(cfg, t, t, counts, offsets, t, t, t, None, ws)
    torch.cuda.synchronize()
    assert (host(counts) == 0).all() and (host(offsets) == 0).all()


@pytest.mark.parametrize("E,T,k,mode", [(256, 16384, 8, 0), (64, 4096, 6, 1), (16, 256, 4, 0), (3, 6, 1, 0)])
def test_bias_update_bit_exact(E, T, k, mode):
    say(f"bias update E={E} T={T} k={k} mode={mode}")
    g = rng(E, T, 7)
    mean = T * k // E
    counts = g.integers(max(0, mean - 3), mean + 4, E).astype(np.int32)
    bias = g.uniform(-0.01, 0.01, E).astype(np.float32)
    cfg = L.make_cfg(T, 128, E, 1, 1, min(k, E), 0, 128, 1, 1.0, "bf16", "bf16", bias_eq_mode=mode)
    b = dev_f32(bias)
    L.moe_update_bias(cfg, dev_i32(counts), b, 1e-3)
    torch.cuda.synchronize()
    exp = oracle.update_bias(bias, counts, T, min(k, E), 1e-3, mode)
    assert (host(b).view(np.uint32) == exp.view(np.uint32)).all()
