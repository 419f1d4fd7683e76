"""The five MoE-layer workloads the layer is exercised on, as plain data.

Shapes follow the DeepSeek-V3 layer the pages describe (hidden 7168, 256 routed
experts, 1 shared expert, 8 routed experts per token, at most 4 nodes per token:
qwbw.cn essay on the DeepSeek-V3 report, section on pre-training, and
DeepSeek-V3 Technical Report：中英对照解读, §2 Architecture).  Group count 8,
intermediate size 2048, the gate scale 2.5, gamma and the input distributions
are not on the pages; they are fixed here as named workloads.

This module holds no arithmetic of the method.  It is shared by the tests, the
benchmark and the C-ABI binding's callers; the oracle does not import it.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int            # tokens in the batch
    H: int            # hidden size
    E: int            # routed experts
    G: int            # expert groups (the one-GPU stand-in for nodes)
    M: int            # groups a token may use
    k: int            # routed experts per token
    S: int            # shared experts
    I: int            # SwiGLU intermediate size per expert
    group_topr: int   # group score = sum of the top-r biased scores in the group
    route_scale: float
    act: str          # "f32" | "bf16"
    wgt: str          # "f32" | "bf16" | "fp8_e4m3"
    sigma: float      # std-dev of every weight tensor
    offset_kind: Optional[str]   # None | "normal" | "zipf"
    zipf_s: float
    bias0_kind: str   # "zero" | "uniform"
    bias0_range: float
    gamma: float
    steps: int
    seed: int = 0
    bias_eq_mode: int = 0

    @property
    def group_size(self) -> int:
        return self.E // self.G

    @property
    def pairs(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "MoeConfig":
        return replace(self, **kw)

    # Algorithmic work counts (what the layer must compute / move).
    def expert_flops(self) -> dict:
        """FLOPs of the routed and shared SwiGLU GEMMs: 3 matmuls of H x I per row."""
        per_row = 2 * 3 * self.H * self.I
        return {"routed": per_row * self.T * self.k, "shared": per_row * self.T * self.S}

    def gate_up_flops(self) -> int:
        """FLOPs of the gate/up GEMMs (routed rows and shared rows)."""
        return 2 * 2 * self.H * self.I * (self.T * self.k + self.T * self.S)

    def down_flops(self) -> int:
        return 2 * self.H * self.I * (self.T * self.k + self.T * self.S)

    def router_flops(self) -> int:
        return 2 * self.T * self.H * self.E


TINY = MoeConfig(
    name="tiny_fp32", T=256, H=128, E=16, G=4, M=2, k=4, S=1, I=64, group_topr=2,
    route_scale=1.0, act="f32", wgt="f32", sigma=0.02, offset_kind="normal", zipf_s=0.0,
    bias0_kind="zero", bias0_range=0.0, gamma=1e-3, steps=10)

MID = MoeConfig(
    name="mid_bf16", T=4096, H=2048, E=64, G=8, M=3, k=6, S=2, I=1408, group_topr=2,
    route_scale=1.0, act="bf16", wgt="bf16", sigma=0.02, offset_kind="zipf", zipf_s=1.1,
    bias0_kind="zero", bias0_range=0.0, gamma=1e-3, steps=50)

V3_PREFILL = MoeConfig(
    name="v3_prefill_bf16", T=16384, H=7168, E=256, G=8, M=4, k=8, S=1, I=2048, group_topr=2,
    route_scale=2.5, act="bf16", wgt="bf16", sigma=0.006, offset_kind=None, zipf_s=0.0,
    bias0_kind="uniform", bias0_range=0.01, gamma=1e-3, steps=1)

V3_DECODE = V3_PREFILL.with_(name="v3_decode_bf16", T=128)

V3_FP8 = V3_PREFILL.with_(name="v3_fp8", T=32768, wgt="fp8_e4m3", offset_kind="zipf",
                          zipf_s=1.5, steps=100)

CONFIGS = {c.name: c for c in (TINY, MID, V3_PREFILL, V3_DECODE, V3_FP8)}
