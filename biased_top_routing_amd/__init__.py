"""MI355X-native DeepSeekMoE layer forward with bias-based (auxiliary-loss-free) balancing.

The compute path is libmoe.so (hand-written HIP kernels for gfx950 behind a
C ABI, include/moe.h); this package holds its sources (csrc/), the build step
(build.py), a ctypes binding with the C names (_lib.py) and a buffer-owning
runner that calls the five entry points in order (runner.py).
"""
from . import _lib  # noqa: F401
from ._lib import (MOE_BF16, MOE_F32, MOE_FFN_ALL, MOE_FFN_DOWN, MOE_FFN_GATE_UP, MOE_FP8_E4M3,  # noqa: F401
                   MOE_SCORES_IN, MOE_WS_DISPATCH, MOE_WS_FFN, MoeCfg, MoeError, MoeExpertWeights, cfg_from,
                   expert_weights, make_cfg, moe_abi_version, moe_combine, moe_dispatch, moe_expert_ffn,
                   moe_quantize_fp8, moe_route, moe_status_string, moe_update_bias, moe_workspace_bytes)
