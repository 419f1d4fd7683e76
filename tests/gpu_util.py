"""Helpers shared by the GPU parity tests (no layer arithmetic here)."""
import sys

import numpy as np
import torch


def say(msg):
    """Name the case before a GPU step, so a failing run tells which case it was."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def host(t) -> np.ndarray:
    """Device tensor -> numpy; bfloat16 comes back as float32 values (exact)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def rel_inf(y, ref) -> float:
    """Normwise max relative error ||y - ref||_inf / ||ref||_inf."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-300))
