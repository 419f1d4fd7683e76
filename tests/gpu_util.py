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


def sample_tokens(T, idx, n, seed, tail=16, per_segment=16):
    """Sorted token rows for sampled output checks: the last `tail` tokens of the batch,
    up to `per_segment` tokens routed to the largest expert segment, and random tokens
    up to `n` in all (every token when T <= n)."""
    if T <= n:
        return np.arange(T)
    idx = np.asarray(idx)
    counts = np.bincount(idx.reshape(-1), minlength=int(idx.max()) + 1)
    big = int(np.argmax(counts))
    in_big = np.flatnonzero((idx == big).any(axis=1))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, T, n])))
    pick = set(range(T - tail, T))
    pick.update(g.choice(in_big, min(per_segment, len(in_big)), replace=False).tolist())
    rest = np.setdiff1d(np.arange(T), np.fromiter(pick, dtype=np.int64))
    pick.update(g.choice(rest, n - len(pick), replace=False).tolist())
    return np.array(sorted(pick))
