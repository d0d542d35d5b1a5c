"""Shared test plumbing: numpy <-> torch device buffers and parity measures."""
from __future__ import annotations

import sys

import numpy as np

import moe_inputs as mi


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    """numpy array -> torch tensor on cuda:0 (uint16 arrays become bfloat16 with the same bits)."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t) -> np.ndarray:
    """torch tensor -> numpy (bfloat16 comes back as uint16 bit patterns)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return mi.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (the layer-output parity measure)."""
    return float(np.abs(as_f64(got) - ref).max() / max(np.abs(ref).max(), 1e-30))


def tolerance(dtype: str) -> float:
    """Output parity bound: 2e-2 of max|y_ref| for bf16 storage, 1e-5 for fp32."""
    return 2e-2 if dtype == "bf16" else 1e-5


def gaps(logits: np.ndarray, K: int):
    """Per token: gap between the K-th and (K+1)-th largest logits, and between the 1st and 2nd."""
    s = -np.sort(-logits, axis=1)
    E = logits.shape[1]
    gapk = s[:, K - 1] - s[:, K] if K < E else np.full(logits.shape[0], np.inf)
    gap12 = s[:, 0] - s[:, 1] if E > 1 else np.full(logits.shape[0], np.inf)
    return gapk, gap12


def selection_is_valid(idx_row: np.ndarray, logits_row: np.ndarray, tol: float) -> bool:
    """A near-tie selection is valid if every kept expert is within tol of every dropped one."""
    kept = set(int(i) for i in idx_row)
    if len(kept) != len(idx_row):
        return False
    dropped = [e for e in range(len(logits_row)) if e not in kept]
    if not dropped:
        return True
    return min(logits_row[list(kept)]) >= max(logits_row[dropped]) - tol
