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


def block_rel_l2(x, ref, blocks):
    """Relative L2 error of every block of a partition of the array, in
    float64: blocks[i] is the block length along axis i (None or missing:
    the whole axis; 1: each index alone); a shorter tail block along an axis
    is a block of its own.  A block whose reference is all zeros is scored by
    its absolute error.  Returns (worst error, start index of the worst block
    per axis)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    blocks = list(blocks) + [None] * (x.ndim - len(blocks))
    pad, shp, lens = [], [], []
    for n, b in zip(x.shape, blocks):
        b = n if (b is None or b >= n) else int(b)
        b = max(b, 1)
        nb = -(-n // b)
        pad.append((0, nb * b - n))
        shp += [nb, b]
        lens.append(b)
    axes = tuple(range(1, 2 * x.ndim, 2))
    d = x - ref
    d *= d
    r2 = ref * ref
    if any(p[1] for p in pad):
        d, r2 = np.pad(d, pad), np.pad(r2, pad)
    d2 = d.reshape(shp).sum(axis=axes)
    r2 = r2.reshape(shp).sum(axis=axes)
    num, den = np.sqrt(d2), np.sqrt(r2)
    err = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    return float(err[i]), tuple(int(j) * b for j, b in zip(i, lens))


def check_blocks(name, x, ref, blocks, tol, errs=None):
    """Assert the whole-array and every block's relative L2 error are within
    tol; record both in errs (name and name + '_blk')."""
    whole = rel_l2(x, ref)
    worst, at = block_rel_l2(x, ref, blocks)
    if errs is not None:
        errs[name] = whole
        errs[name + "_blk"] = worst
    assert whole <= tol, (name, whole)
    assert worst <= tol, (name, "block", at, worst)
    return whole, worst


# Blocks for the chunkwise outputs of sampled sequences ([n, T, d], [n, T] or
# [n, T, DK] per token; [n, DK, DV] per state): 1024 tokens of one sequence
# (the longest backward segment), and each sequence's state on its own.
CHUNK_BLOCKS = {"o": (1, 1024), "dq": (1, 1024), "dk": (1, 1024), "dv": (1, 1024),
                "dl": (1, 1024), "ST": (1,), "dS0": (1,)}


def say(*a):
    """Print a progress line that names the case, flushed before the GPU runs it."""
    print(*a, flush=True)
    sys.stdout.flush()
