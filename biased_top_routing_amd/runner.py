"""Device buffers for one MoE layer and the five C-ABI calls in order.

MoeLayerGPU uploads a layer's weights once, allocates every buffer the calls
need for T tokens, and runs route -> dispatch -> expert FFN -> combine ->
bias update on the current stream.  It only allocates and marshals; every step
of the layer runs in libmoe's kernels.  With gather=True, dispatch writes only
the indices and the routed gate/up GEMM reads its rows from x through perm
(moe_expert_ffn_gather); no x_perm is allocated.  With save_gu=True (bf16),
the forward pass keeps the gate and up outputs (moe_expert_ffn_save) and the
backward pass starts from them (moe_expert_ffn_backward_saved) instead of
recomputing the gate/up GEMM.  With keep_scores=False, moe_route writes no
[T, E] affinities (a forward pass that needs no router gradient).
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def to_device(arr, device="cuda"):
    """numpy float32 -> float32 tensor; numpy uint16 (bf16 bit patterns) -> bfloat16 tensor."""
    if arr is None:
        return None
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


class MoeLayerGPU:
    def __init__(self, cfg, weights, T=None, device="cuda", gather=False, save_gu=False, keep_scores=True):
        self.c = cfg
        self.device = device
        self.gather = gather
        self.save_gu = save_gu
        self.keep_scores = keep_scores
        self.fp8 = cfg.wgt == "fp8_e4m3"
        self.act_dtype = torch.float32 if cfg.act == "f32" else torch.bfloat16
        dev = lambda a: to_device(a, device)
        self.w_router = dev(weights.w_router)
        self.logit_offset = dev(weights.logit_offset)
        if self.fp8:
            self.w_gate_up, self.w_gate_up_scale = self._quantize(weights.w_gate_up)
            self.w_down, self.w_down_scale = self._quantize(weights.w_down)
            self.ws_gate_up, self.ws_gate_up_scale = self._quantize(weights.ws_gate_up)
            self.ws_down, self.ws_down_scale = self._quantize(weights.ws_down)
        else:
            self.w_gate_up, self.w_down = dev(weights.w_gate_up), dev(weights.w_down)
            self.ws_gate_up, self.ws_down = dev(weights.ws_gate_up), dev(weights.ws_down)
            self.w_gate_up_scale = self.w_down_scale = self.ws_gate_up_scale = self.ws_down_scale = None
        self.weights = L.expert_weights(self.w_gate_up, self.w_down, self.ws_gate_up, self.ws_down,
                                        self.w_gate_up_scale, self.w_down_scale, self.ws_gate_up_scale,
                                        self.ws_down_scale)
        self.alloc(cfg.T if T is None else T)

    def _quantize(self, w_np):
        """bf16 weights [n, rows, cols] -> E4M3 codes + one fp32 scale per 128 x 128 block (on the GPU)."""
        n, rows, cols = w_np.shape
        codes = torch.empty((n, rows, cols), dtype=torch.uint8, device=self.device)
        scales = torch.empty((n, rows // 128, cols // 128), dtype=torch.float32, device=self.device)
        if n:
            src = to_device(w_np, self.device)
            L.moe_quantize_fp8(src, n, rows, cols, 128, codes, scales)
            torch.cuda.current_stream().synchronize()
            del src
        return codes, scales

    def alloc(self, T):
        c = self.c
        self.T = T
        self.cfg = L.cfg_from(c, T=T)
        d, P = self.device, T * c.k
        f32, i32 = torch.float32, torch.int32
        # the [T, E] affinities (the backward pass reads them); without them moe_route
        # gets a workspace instead and a fused router kernel keeps them on chip
        self.scores = torch.empty((T, c.E), dtype=f32, device=d)
        self.ws_route = torch.empty(L.moe_workspace_bytes(self.cfg, L.MOE_WS_ROUTE), dtype=torch.uint8, device=d)
        self.topk_idx = torch.empty((T, c.k), dtype=i32, device=d)
        self.topk_w = torch.empty((T, c.k), dtype=f32, device=d)
        self.counts = torch.empty(c.E, dtype=i32, device=d)
        self.offsets = torch.empty(c.E + 1, dtype=i32, device=d)
        self.perm = torch.empty(P, dtype=i32, device=d)
        self.inv = torch.empty((T, c.k), dtype=i32, device=d)
        if self.gather:
            self.x_perm = self.x_perm_scale = None
        elif self.fp8:
            self.x_perm = torch.empty((P, c.H), dtype=torch.uint8, device=d)
            self.x_perm_scale = torch.empty((P, c.H // 128), dtype=f32, device=d)
        else:
            self.x_perm = torch.empty((P, c.H), dtype=self.act_dtype, device=d)
            self.x_perm_scale = None
        self.y_perm = torch.empty((P, c.H), dtype=self.act_dtype, device=d)
        self.y_shared = torch.empty((T, c.H), dtype=self.act_dtype, device=d) if c.S > 0 else None
        self.y = torch.empty((T, c.H), dtype=self.act_dtype, device=d)
        self.ws_dispatch = torch.empty(L.moe_workspace_bytes(self.cfg, L.MOE_WS_DISPATCH), dtype=torch.uint8,
                                       device=d)
        self.ws_ffn = torch.empty(L.moe_workspace_bytes(self.cfg, L.MOE_WS_FFN), dtype=torch.uint8, device=d)
        if self.save_gu:
            bf = torch.bfloat16
            self.g = torch.empty((P, c.I), dtype=bf, device=d)
            self.u = torch.empty((P, c.I), dtype=bf, device=d)
            self.gs = torch.empty((T, c.S * c.I), dtype=bf, device=d) if c.S > 0 else None
            self.us = torch.empty((T, c.S * c.I), dtype=bf, device=d) if c.S > 0 else None
            self.saved = L.ffn_saved(self.g, self.u, self.gs, self.us)

    # ---------------------------------------------------------------- the five calls
    def route(self, x, bias, scores_in=False):
        keep = self.keep_scores or scores_in
        L.moe_route(self.cfg, x, self.w_router, self.logit_offset, bias, self.scores if keep else None,
                    L.MOE_SCORES_IN if scores_in else 0, self.topk_idx, self.topk_w,
                    None if keep else self.ws_route)

    def dispatch(self, x):
        L.moe_dispatch(self.cfg, self.topk_idx, x, self.counts, self.offsets, self.perm, self.inv, self.x_perm,
                       self.x_perm_scale, self.ws_dispatch)

    def expert_ffn(self, x, phase=L.MOE_FFN_ALL):
        if self.save_gu:
            L.moe_expert_ffn_save(self.cfg, self.x_perm, self.perm, self.offsets, self.weights, x, self.y_perm,
                                  self.y_shared, self.saved, self.ws_ffn, phase)
        elif self.gather:
            L.moe_expert_ffn_gather(self.cfg, x, self.perm, self.offsets, self.weights, self.y_perm,
                                    self.y_shared, self.ws_ffn, phase)
        else:
            L.moe_expert_ffn(self.cfg, self.x_perm, self.x_perm_scale, self.offsets, self.weights, x,
                             self.y_perm, self.y_shared, self.ws_ffn, phase)

    def combine(self):
        L.moe_combine(self.cfg, self.y_perm, self.y_shared, self.inv, self.topk_w, self.y)

    def update_bias(self, bias, gamma):
        L.moe_update_bias(self.cfg, self.counts, bias, gamma)

    # ---------------------------------------------------------------- backward
    def alloc_backward(self):
        """Gradient buffers for the current T (fp32 weight gradients, bf16 activation gradients)."""
        c, d = self.c, self.device
        T, P = self.T, self.T * c.k
        bf, f32 = torch.bfloat16, torch.float32
        self.dy_perm = torch.empty((P, c.H), dtype=bf, device=d)
        self.d_topk_w = torch.empty((T, c.k), dtype=f32, device=d)
        self.dx_perm = torch.empty((P, c.H), dtype=bf, device=d)
        self.dx_shared = torch.empty((T, c.H), dtype=bf, device=d) if c.S > 0 else None
        self.dx_router = torch.empty((T, c.H), dtype=f32, device=d)
        self.dx = torch.empty((T, c.H), dtype=bf, device=d)
        self.g_w_gate_up = torch.empty((c.E, 2 * c.I, c.H), dtype=f32, device=d)
        self.g_w_down = torch.empty((c.E, c.H, c.I), dtype=f32, device=d)
        self.g_ws_gate_up = torch.empty((c.S, 2 * c.I, c.H), dtype=f32, device=d) if c.S > 0 else None
        self.g_ws_down = torch.empty((c.S, c.H, c.I), dtype=f32, device=d) if c.S > 0 else None
        self.g_w_router = torch.empty((c.E, c.H), dtype=f32, device=d)
        self.loss_bal = torch.empty(1, dtype=f32, device=d)
        self.grads = L.expert_grads(self.g_w_gate_up, self.g_w_down, self.g_ws_gate_up, self.g_ws_down)
        self.ws_ffn_bwd = torch.empty(L.moe_workspace_bytes(self.cfg, L.MOE_WS_FFN_BWD), dtype=torch.uint8, device=d)
        self.ws_route_bwd = torch.empty(L.moe_workspace_bytes(self.cfg, L.MOE_WS_ROUTE_BWD), dtype=torch.uint8,
                                        device=d)
        self._bwd_T = T

    def backward(self, x, dy, alpha=0.0, seq_len=0):
        """Gradients of sum(dy * y) + alpha-weighted sequence balance loss for the last forward pass
        (same x, same routing).  Fills dx, the fp32 weight gradients and loss_bal; returns dx."""
        if self.gather:
            raise ValueError("backward reads the permuted rows x_perm: build the layer with gather=False")
        if getattr(self, "_bwd_T", None) != self.T:
            self.alloc_backward()
        cfg = self.cfg
        L.moe_combine_backward(cfg, dy, self.y_perm, self.inv, self.topk_w, self.dy_perm, self.d_topk_w)
        if self.save_gu:
            L.moe_expert_ffn_backward_saved(cfg, self.x_perm, x, self.offsets, self.weights, self.saved, self.dy_perm,
                                            dy, self.dx_perm, self.dx_shared, self.grads, self.ws_ffn_bwd)
        else:
            L.moe_expert_ffn_backward(cfg, self.x_perm, x, self.offsets, self.weights, self.dy_perm, dy,
                                      self.dx_perm, self.dx_shared, self.grads, self.ws_ffn_bwd)
        L.moe_route_backward(cfg, x, self.w_router, self.scores, self.topk_idx, self.d_topk_w, alpha, seq_len,
                             self.dx_router, self.g_w_router, self.loss_bal, self.ws_route_bwd)
        L.moe_dispatch_backward(cfg, self.dx_perm, self.dx_shared, self.dx_router, self.inv, self.dx)
        return self.dx

    def forward(self, x, bias, gamma=None, scores_in=False):
        """One batch through the layer; with gamma set, bias is updated in place afterwards."""
        self.route(x, bias, scores_in)
        self.dispatch(x)
        self.expert_ffn(x)
        self.combine()
        if gamma is not None:
            self.update_bias(bias, gamma)
        return self.y

    # ---------------------------------------------------------------- HIP graph
    def capture(self, x, bias, gamma=None):
        """Record one forward() over the tensors x and bias (and the bias update when
        gamma is set) into a HIP graph; replay() reruns it on whatever they then hold.
        One graph serves every batch of this T: each launch is sized by capacity (the
        grouped GEMMs' tile tables are built on the device from the batch's routing)
        and no call allocates, copies or synchronises, so the recorded work is the
        same kernels forward() launches.  A warm-up pass (no bias update) on a side
        stream precedes the capture."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.forward(x, bias, None)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.forward(x, bias, gamma)
        self.graph_inputs = (x, bias)
        return self.graph

    def replay(self):
        """One replay of the captured step on the current stream; returns y."""
        self.graph.replay()
        return self.y
