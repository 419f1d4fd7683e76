"""GPU: the routed gate/up GEMM reading its rows straight from x through perm
(moe_expert_ffn_gather, with moe_dispatch writing indices only) against the
materialised x_perm path.

Both paths multiply the same rows in the same order with the same kernels, so
routing, counts, offsets, perm, inv, h, y_perm, y_shared and y must agree bit for
bit; the layer output of the gather path is also checked against the oracle at
the same bounds as the materialised path.  Cases span fp32, bf16 (large tiles,
ragged segments, empty experts from a Zipf skew, two shared experts, no shared
expert), the small-batch bf16 tiles and FP8 with and without a shared expert."""
import numpy as np
import pytest
import torch

import oracle
from biased_top_routing_amd import _lib as L
from biased_top_routing_amd.runner import MoeLayerGPU, to_device
from gpu_util import host, rel_inf, say
from workloads import MID, TINY
from workloads.inputs import make_weights, make_x

pytestmark = pytest.mark.gpu

FP8 = dict(H=256, E=16, G=4, M=2, k=4, I=256, wgt="fp8_e4m3", group_topr=2)
CASES = {
    "tiny_f32": (TINY, 1e-4),
    "bf16_ragged_S2": (MID.with_(T=1000, H=512, E=64, I=256, S=2), 2e-2),
    "bf16_zipf_S0": (MID.with_(T=700, H=256, E=64, I=128, S=0), 2e-2),
    "bf16_small_batch": (MID.with_(T=40, H=512, E=64, I=256, S=1), 2e-2),
    "fp8_S1": (MID.with_(T=300, S=1, **FP8), 6e-2),
    "fp8_S0": (MID.with_(T=517, S=0, **FP8), 6e-2),
}


def _bits(t):
    """Device tensor -> its raw bits on the host (exact comparison, NaN-safe)."""
    if t is None:
        return None
    t = t.detach().contiguous()
    view = {torch.float32: torch.int32, torch.bfloat16: torch.int16}.get(t.dtype)
    return (t.view(view) if view is not None else t).cpu().numpy()


def _h_bits(layer):
    off, n = L.moe_ffn_workspace_part(layer.cfg, L.MOE_WSP_H)
    return layer.ws_ffn[off:off + n].cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_gather_matches_materialised(name):
    c, tol = CASES[name]
    w = make_weights(c)
    xh = make_x(c)
    x = to_device(xh)
    say(f"gather {name}: materialised path")
    ref = MoeLayerGPU(c, w)
    bias = torch.from_numpy(w.bias0.copy()).cuda()
    ref.forward(x, bias)
    torch.cuda.synchronize()
    say(f"gather {name}: gathered path")
    g = MoeLayerGPU(c, w, gather=True)
    assert g.x_perm is None
    bias_g = torch.from_numpy(w.bias0.copy()).cuda()
    g.forward(x, bias_g)
    torch.cuda.synchronize()
    for f in ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv"):
        assert (_bits(getattr(ref, f)) == _bits(getattr(g, f))).all(), f
    assert (_h_bits(ref) == _h_bits(g)).all(), "h"
    assert (_bits(ref.y_perm) == _bits(g.y_perm)).all(), "y_perm"
    if c.S > 0:
        assert (_bits(ref.y_shared) == _bits(g.y_shared)).all(), "y_shared"
    assert (_bits(ref.y) == _bits(g.y)).all(), "y"
    # and the oracle, teacher-forced on the GPU's routing
    s = host(g.scores)
    idx = host(g.topk_idx)
    idx_o, w_o = oracle.route(s, w.bias0, c.G, c.M, c.k, c.group_topr, c.route_scale)
    assert (idx == idx_o).all()
    if c.wgt == "fp8_e4m3":
        o = oracle.forward_from_routing(c, xh, w, w.bias0, s, idx, w_o)
    else:
        x64 = oracle.decode_act(xh).astype(np.float64)
        s_o = oracle.affinity(x64, oracle.decode_act(w.w_router), w.logit_offset).astype(np.float64)
        sel = np.take_along_axis(s_o, idx.astype(np.int64), 1)
        o = oracle.forward_from_routing(c, xh, w, w.bias0, s_o.astype(np.float32), idx,
                                        c.route_scale * sel / sel.sum(1, keepdims=True))
    err = rel_inf(host(g.y), o["y"])
    say(f"gather {name}: layer error {err:.2e}")
    assert err < tol
