"""Shared helpers for the GPU parity tests (not collected by pytest)."""

import sys

import numpy as np
import torch


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def to_dev(x, dtype=None):
    """numpy -> device tensor; uint16 arrays become bf16 (same bits)."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dev())


def to_np(t):
    """device tensor -> numpy float64 (bf16 upcast exactly)."""
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return num
    return num / den


def say(*a):
    """Print a progress line that names the case, flushed before the GPU runs it."""
    print(*a, flush=True)
    sys.stdout.flush()
