"""moe_dispatch_noalloc (dispatch with the library's fixed device scratch instead of a
workspace) against moe_dispatch on the same inputs, bit for bit, over calls in a row
whose sizes shrink (the scratch keeps the previous call's contents), including the FP8
quantising row copy and the indices-only form; and against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from biased_top_routing_amd import _lib as L
from gpu_util import dev_i32, host, say
from workloads.inputs import f32_to_bf16_bits, rng

pytestmark = pytest.mark.gpu

CASES = [
    # (T, H, E, G, M, k, wgt, rows copied)
    (5000, 512, 256, 8, 4, 8, "bf16", True),
    (1500, 256, 64, 8, 3, 6, "fp8_e4m3", True),
    (77, 128, 16, 4, 2, 4, "bf16", False),
]


def _dispatch(fn, cfg, idx, x, T, H, k, fp8, copy):
    P = T * k
    out = {n: torch.full(shape, -7, dtype=torch.int32, device="cuda")
           for n, shape in (("counts", (cfg.E,)), ("offsets", (cfg.E + 1,)), ("perm", (P,)), ("inv", (T, k)))}
    xp = xs = None
    if copy:
        xp = torch.empty((P, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
        xs = torch.empty((P, H // 128), dtype=torch.float32, device="cuda") if fp8 else None
    args = (cfg, idx, x, out["counts"], out["offsets"], out["perm"], out["inv"], xp, xs)
    if fn == "noalloc":
        L.moe_dispatch_noalloc(*args)
    else:
        ws = torch.empty(L.moe_workspace_bytes(cfg, L.MOE_WS_DISPATCH), dtype=torch.uint8, device="cuda")
        L.moe_dispatch(*args, ws)
    torch.cuda.synchronize()
    res = {n: host(t) for n, t in out.items()}
    if copy:
        res["x_perm"] = xp.view(torch.uint8).cpu().numpy() if fp8 else xp.view(torch.int16).cpu().numpy()
        if fp8:
            res["x_perm_scale"] = host(xs).view(np.uint32)
    return res


def test_dispatch_noalloc_matches_dispatch():
    for T, H, E, G, M, k, wgt, copy in CASES:
        say(f"dispatch without workspace T={T} H={H} E={E} k={k} {wgt} copy={copy}")
        cfg = L.make_cfg(T, H, E, G, M, k, 0, 128, 2, 1.0, "bf16", wgt)
        g = rng(T, E, 3)
        idx = np.argsort(-g.random((T, E)), axis=1)[:, :k].astype(np.int32)
        xb = f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        fp8 = wgt == "fp8_e4m3"
        a = _dispatch("noalloc", cfg, dev_i32(idx), x, T, H, k, fp8, copy)
        b = _dispatch("ws", cfg, dev_i32(idx), x, T, H, k, fp8, copy)
        assert a.keys() == b.keys()
        for n in a:
            assert (a[n] == b[n]).all(), n
        c_o, o_o, p_o, i_o = oracle.dispatch(idx, E)
        assert (a["counts"] == c_o).all() and (a["offsets"] == o_o).all()
        assert (a["perm"] == p_o).all() and (a["inv"] == i_o).all()


def test_dispatch_noalloc_rejects_sizes_beyond_its_scratch():
    # ceil(T*k / 1024) * E * 4 bytes > 4 MiB: 4097 segments of 256 experts
    cfg = L.make_cfg(524416, 128, 256, 8, 4, 8, 0, 128, 2, 1.0, "bf16", "bf16")
    t = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(L.MoeError) as e:
        L.moe_dispatch_noalloc(cfg, t, None, t, t, t, t, None, None)
    assert e.value.status == L.MOE_ERR_SCRATCH
