"""Named MoE-layer workloads and their seeded synthetic inputs (no layer arithmetic)."""
from .configs import CONFIGS, MID, TINY, V3_DECODE, V3_FP8, V3_PREFILL, MoeConfig  # noqa: F401
