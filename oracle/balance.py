"""Oracle: the per-step bias update of auxiliary-loss-free balancing.

TEST INFRASTRUCTURE (see the package docstring).

After each step the load of every expert over the whole batch is compared with
the balanced load; an overloaded expert's bias falls by gamma and an
underloaded expert's bias rises by gamma (reading notes, Method §1
"Auxiliary-loss-free 负载均衡"; qwbw.cn essay, load-balancing section;
DeepSeek-V3 Technical Report：中英对照解读, §3).

Readings: "overloaded" means load > T*k/E (compared exactly as load*E > T*k);
an expert at exactly the mean counts as underloaded (mode 0), so every bias
moves by exactly gamma each step; mode 1 leaves it unchanged instead.  The
arithmetic is one fp32 add (round to nearest even) with gamma = fl32(gamma).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def update_bias(bias: np.ndarray, counts: np.ndarray, n_tokens: int, top_k: int,
                gamma: float, eq_mode: int = 0) -> np.ndarray:
    b = np.asarray(bias, F32)
    c = np.asarray(counts, np.int64)
    E = b.shape[0]
    total = int(n_tokens) * int(top_k)
    over = c * E > total
    under = (c * E <= total) if eq_mode == 0 else (c * E < total)
    g = F32(gamma)
    out = b.copy()
    out[over] = (b[over] - g).astype(F32)
    out[under] = (b[under] + g).astype(F32)
    return out
