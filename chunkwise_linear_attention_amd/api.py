"""Torch-facing wrappers with the same names as the C ABI calls.

Each wrapper checks dtypes, devices and shapes, allocates the outputs and the
workspace with torch, and calls the library on torch's current stream.
"""

from __future__ import annotations

import torch

from . import _lib

CHUNK = 64


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opt(t, *a):
    if t is not None:
        _need(t, *a)


def _workspace(nbytes, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


# ---------------------------------------------------------------------------
# log-decay checks
# ---------------------------------------------------------------------------

_CHECK_INPUTS = False


def set_input_checks(on: bool) -> bool:
    """With on=True, chunked_linear_attn[_bwd] and gla[_bwd] first run
    check_log_decay on their log decays (a pass over the tensor and a
    synchronization; off by default).  Returns the previous setting."""
    global _CHECK_INPUTS
    prev, _CHECK_INPUTS = _CHECK_INPUTS, bool(on)
    return prev


def log_decay_counts(log_decay) -> dict:
    """Numbers of NaN, +inf, finite positive and -inf values in a fp32 device
    tensor, counted on the device (cla_check_log_decay)."""
    if not isinstance(log_decay, torch.Tensor) or log_decay.dtype != torch.float32:
        raise TypeError("log_decay must be a float32 torch.Tensor")
    if not log_decay.is_contiguous():
        raise ValueError("log_decay must be contiguous")
    dev = log_decay.device
    counts = torch.empty(4, dtype=torch.int32, device=dev)
    st = _lib.lib().cla_check_log_decay(_ptr(log_decay), log_decay.numel(), _ptr(counts),
                                        _stream(dev))
    _lib.check("cla_check_log_decay", st)
    c = [int(x) & 0xFFFFFFFF for x in counts.cpu().tolist()]
    return {"nan": c[0], "posinf": c[1], "positive": c[2], "neginf": c[3]}


def check_log_decay(log_decay, kind: str = "scalar") -> None:
    """Raise ValueError if log_decay holds values the chunkwise calls do not
    accept: NaN or +inf for the scalar decay (kind="scalar"); anything but
    finite values <= 0 for one decay per key dimension (kind="gla")."""
    if kind not in ("scalar", "gla"):
        raise ValueError("kind must be 'scalar' or 'gla'")
    c = log_decay_counts(log_decay)
    bad = ("nan", "posinf") if kind == "scalar" else ("nan", "posinf", "positive", "neginf")
    found = {k: c[k] for k in bad if c[k]}
    if found:
        rule = ("finite or -inf" if kind == "scalar" else "finite and <= 0")
        raise ValueError(f"log_decay must be {rule}; found " +
                         ", ".join(f"{v} {k}" for k, v in found.items()))


# ---------------------------------------------------------------------------
# diagonal scan
# ---------------------------------------------------------------------------


def scan_workspace_bytes(B: int, T: int, D: int) -> int:
    return int(_lib.lib().cla_scan_workspace_bytes(B, T, D))


def scan(a, b, h0=None, *, want_final=True, workspace=None):
    """h_t = a_t h_{t-1} + b_t over dim 1 of [B, T, D] fp32 tensors.
    Returns (h, h_T) (h_T is None when want_final is False)."""
    if a.dim() != 3:
        raise ValueError("a must be [B, T, D]")
    B, T, D = a.shape
    dev = a.device
    _need(a, "a", torch.float32, (B, T, D), dev)
    _need(b, "b", torch.float32, (B, T, D), dev)
    _opt(h0, "h0", torch.float32, (B, D), dev)
    h = torch.empty_like(a)
    hT = torch.empty((B, D), dtype=torch.float32, device=dev) if want_final else None
    L = _lib.lib()
    nbytes = int(L.cla_scan_workspace_bytes(B, T, D))
    if workspace is None:
        ws, wsb = _workspace(nbytes, dev)
    else:
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    st = L.cla_scan_fwd(_ptr(a), _ptr(b), _ptr(h0), _ptr(h), _ptr(hT), B, T, D,
                        _ptr(ws), wsb, _stream(dev))
    _lib.check("cla_scan_fwd", st)
    return h, hT


def scan_fwd_noalloc(a, b, h0, h, hT=None):
    """``scan`` for callers that cannot allocate: the outputs h [B, T, D] and
    hT [B, D] (or None) are the caller's, and the library keeps the segment
    pairs in its own fixed device array, so nothing is allocated here or in
    the library.  Calls that may overlap on one GPU must be ordered."""
    if a.dim() != 3:
        raise ValueError("a must be [B, T, D]")
    B, T, D = a.shape
    dev = a.device
    _need(a, "a", torch.float32, (B, T, D), dev)
    _need(b, "b", torch.float32, (B, T, D), dev)
    _opt(h0, "h0", torch.float32, (B, D), dev)
    _need(h, "h", torch.float32, (B, T, D), dev)
    _opt(hT, "hT", torch.float32, (B, D), dev)
    st = _lib.lib().cla_scan_fwd_noalloc(_ptr(a), _ptr(b), _ptr(h0), _ptr(h), _ptr(hT),
                                         B, T, D, _stream(dev))
    _lib.check("cla_scan_fwd_noalloc", st)
    return h, hT


def scan_bwd(a, h, h0, dh, dhT=None, *, want_dh0=True, workspace=None):
    """Backward of ``scan``: returns (da, db, dh0)."""
    B, T, D = a.shape
    dev = a.device
    _need(a, "a", torch.float32, (B, T, D), dev)
    _need(h, "h", torch.float32, (B, T, D), dev)
    _opt(h0, "h0", torch.float32, (B, D), dev)
    _need(dh, "dh", torch.float32, (B, T, D), dev)
    _opt(dhT, "dhT", torch.float32, (B, D), dev)
    da = torch.empty_like(a)
    db = torch.empty_like(a)
    dh0 = torch.empty((B, D), dtype=torch.float32, device=dev) if want_dh0 else None
    L = _lib.lib()
    nbytes = int(L.cla_scan_workspace_bytes(B, T, D))
    if workspace is None:
        ws, wsb = _workspace(nbytes, dev)
    else:
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    st = L.cla_scan_bwd(_ptr(a), _ptr(h), _ptr(h0), _ptr(dh), _ptr(dhT), _ptr(da),
                        _ptr(db), _ptr(dh0), B, T, D, _ptr(ws), wsb, _stream(dev))
    _lib.check("cla_scan_bwd", st)
    return da, db, dh0


# ---------------------------------------------------------------------------
# chunkwise linear attention
# ---------------------------------------------------------------------------


def chunk_workspace_bytes(B, H, T, DK, DV, backward=False, chunk=CHUNK) -> int:
    return int(_lib.lib().cla_chunk_workspace_bytes(B, H, T, DK, DV, chunk, int(backward)))


def chunk_saved_bytes(B, H, T, DK, DV, chunk=CHUNK) -> int:
    return int(_lib.lib().cla_chunk_saved_bytes(B, H, T, DK, DV, chunk))


def chunked_linear_attn(q, k, v, log_decay, S0=None, *, want_final=True,
                        chunk=CHUNK, workspace=None, save_states=False):
    """S_t = exp(l_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, chunkwise.
    q, k: [B, H, T, DK] bf16; v: [B, H, T, DV] bf16; log_decay: [B, H, T] fp32;
    S0: [B, H, DK, DV] fp32 or None.  Returns (o bf16, S_T fp32 or None), and
    with save_states=True also the saved segment states for
    ``chunked_linear_attn_bwd(..., saved=...)`` (cla_chunk_fwd_saved)."""
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, H, T, DK), dev)
    _need(k, "k", torch.bfloat16, (B, H, T, DK), dev)
    _need(v, "v", torch.bfloat16, (B, H, T, DV), dev)
    _need(log_decay, "log_decay", torch.float32, (B, H, T), dev)
    if _CHECK_INPUTS:
        check_log_decay(log_decay, "scalar")
    _opt(S0, "S0", torch.float32, (B, H, DK, DV), dev)
    o = torch.empty((B, H, T, DV), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev) if want_final else None
    L = _lib.lib()
    nbytes = int(L.cla_chunk_workspace_bytes(B, H, T, DK, DV, chunk, 0))
    if workspace is None:
        ws, wsb = _workspace(nbytes, dev)
    else:
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    if not save_states:
        st = L.cla_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S0), _ptr(o),
                             _ptr(ST), B, H, T, DK, DV, chunk, _ptr(ws), wsb, _stream(dev))
        _lib.check("cla_chunk_fwd", st)
        return o, ST
    sb = int(L.cla_chunk_saved_bytes(B, H, T, DK, DV, chunk))
    saved = torch.empty(max(sb, 1), dtype=torch.uint8, device=dev)
    st = L.cla_chunk_fwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S0), _ptr(o),
                               _ptr(ST), _ptr(saved), saved.numel(), B, H, T, DK, DV, chunk,
                               _ptr(ws), wsb, _stream(dev))
    _lib.check("cla_chunk_fwd_saved", st)
    return o, ST, saved


def chunked_linear_attn_bwd(q, k, v, log_decay, S0, dO, dST=None, *, want_dS0=True,
                            chunk=CHUNK, workspace=None, saved=None):
    """Backward of ``chunked_linear_attn``: returns (dq, dk, dv, dlog_decay, dS0).
    ``saved``: the states returned by the forward with save_states=True
    (cla_chunk_bwd_saved), or None (cla_chunk_bwd)."""
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, H, T, DK), dev)
    _need(k, "k", torch.bfloat16, (B, H, T, DK), dev)
    _need(v, "v", torch.bfloat16, (B, H, T, DV), dev)
    _need(log_decay, "log_decay", torch.float32, (B, H, T), dev)
    if _CHECK_INPUTS:
        check_log_decay(log_decay, "scalar")
    _opt(S0, "S0", torch.float32, (B, H, DK, DV), dev)
    _need(dO, "dO", torch.bfloat16, (B, H, T, DV), dev)
    _opt(dST, "dST", torch.float32, (B, H, DK, DV), dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dl = torch.empty_like(log_decay)
    dS0 = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev) if want_dS0 else None
    L = _lib.lib()
    nbytes = int(L.cla_chunk_workspace_bytes(B, H, T, DK, DV, chunk, 1))
    if workspace is None:
        ws, wsb = _workspace(nbytes, dev)
    else:
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    if saved is None:
        st = L.cla_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S0), _ptr(dO),
                             _ptr(dST), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dl), _ptr(dS0),
                             B, H, T, DK, DV, chunk, _ptr(ws), wsb, _stream(dev))
        _lib.check("cla_chunk_bwd", st)
    else:
        if saved.device != dev:
            raise ValueError("saved must be on the same device as q")
        st = L.cla_chunk_bwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S0),
                                   _ptr(dO), _ptr(dST), _ptr(saved),
                                   saved.numel() * saved.element_size(), _ptr(dq), _ptr(dk),
                                   _ptr(dv), _ptr(dl), _ptr(dS0), B, H, T, DK, DV, chunk,
                                   _ptr(ws), wsb, _stream(dev))
        _lib.check("cla_chunk_bwd_saved", st)
    return dq, dk, dv, dl, dS0


# ---------------------------------------------------------------------------
# one decay per key dimension (gated linear attention)
# ---------------------------------------------------------------------------


def gla_workspace_bytes(B, H, T, DK, DV, backward=False, chunk=CHUNK) -> int:
    return int(_lib.lib().cla_gla_workspace_bytes(B, H, T, DK, DV, chunk, int(backward)))


def gla_saved_bytes(B, H, T, DK, DV, chunk=CHUNK) -> int:
    return int(_lib.lib().cla_gla_saved_bytes(B, H, T, DK, DV, chunk))


def gla(q, k, v, log_decay, S0=None, *, want_final=True, chunk=CHUNK, workspace=None,
        save_states=False):
    """S_t = diag(exp(l_t)) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, chunkwise, with
    one log decay per key dimension.  q, k: [B, H, T, DK] bf16; v: [B, H, T, DV]
    bf16; log_decay: [B, H, T, DK] fp32; S0: [B, H, DK, DV] fp32 or None.
    Returns (o bf16, S_T fp32 or None), and with save_states=True also the
    saved segment start states for ``gla_bwd(..., saved=...)``
    (cla_gla_fwd_saved)."""
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, H, T, DK), dev)
    _need(k, "k", torch.bfloat16, (B, H, T, DK), dev)
    _need(v, "v", torch.bfloat16, (B, H, T, DV), dev)
    _need(log_decay, "log_decay", torch.float32, (B, H, T, DK), dev)
    if _CHECK_INPUTS:
        check_log_decay(log_decay, "gla")
    _opt(S0, "S0", torch.float32, (B, H, DK, DV), dev)
    o = torch.empty((B, H, T, DV), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev) if want_final else None
    L = _lib.lib()
    nbytes = int(L.cla_gla_workspace_bytes(B, H, T, DK, DV, chunk, 0))
    if workspace is None:
        ws, wsb = _workspace(nbytes, dev)
    else:
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    if not save_states:
        st = L.cla_gla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S0), _ptr(o),
                           _ptr(ST), B, H, T, DK, DV, chunk, _ptr(ws), wsb, _stream(dev))
        _lib.check("cla_gla_fwd", st)
        return o, ST
    sb = int(L.cla_gla_saved_bytes(B, H, T, DK, DV, chunk))
    saved = torch.empty(max(sb, 1), dtype=torch.uint8, device=dev)
    st = L.cla_gla_fwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S0), _ptr(o),
                             _ptr(ST), _ptr(saved), saved.numel(), B, H, T, DK, DV, chunk,
                             _ptr(ws), wsb, _stream(dev))
    _lib.check("cla_gla_fwd_saved", st)
    return o, ST, saved


def gla_bwd(q, k, v, log_decay, S0, dO, dST=None, *, want_dS0=True, chunk=CHUNK,
            workspace=None, saved=None):
    """Backward of ``gla``: returns (dq, dk, dv, dlog_decay [B, H, T, DK], dS0).
    ``saved``: the states returned by the forward with save_states=True
    (cla_gla_bwd_saved), or None (cla_gla_bwd)."""
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, H, T, DK), dev)
    _need(k, "k", torch.bfloat16, (B, H, T, DK), dev)
    _need(v, "v", torch.bfloat16, (B, H, T, DV), dev)
    _need(log_decay, "log_decay", torch.float32, (B, H, T, DK), dev)
    if _CHECK_INPUTS:
        check_log_decay(log_decay, "gla")
    _opt(S0, "S0", torch.float32, (B, H, DK, DV), dev)
    _need(dO, "dO", torch.bfloat16, (B, H, T, DV), dev)
    _opt(dST, "dST", torch.float32, (B, H, DK, DV), dev)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dl = torch.empty_like(log_decay)
    dS0 = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev) if want_dS0 else None
    L = _lib.lib()
    nbytes = int(L.cla_gla_workspace_bytes(B, H, T, DK, DV, chunk, 1))
    if workspace is None:
        ws, wsb = _workspace(nbytes, dev)
    else:
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    if saved is None:
        st = L.cla_gla_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S0), _ptr(dO),
                           _ptr(dST), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dl), _ptr(dS0),
                           B, H, T, DK, DV, chunk, _ptr(ws), wsb, _stream(dev))
        _lib.check("cla_gla_bwd", st)
    else:
        if saved.device != dev:
            raise ValueError("saved must be on the same device as q")
        st = L.cla_gla_bwd_saved(_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(S0),
                                 _ptr(dO), _ptr(dST), _ptr(saved),
                                 saved.numel() * saved.element_size(), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(dl), _ptr(dS0), B, H, T, DK, DV, chunk,
                                 _ptr(ws), wsb, _stream(dev))
        _lib.check("cla_gla_bwd_saved", st)
    return dq, dk, dv, dl, dS0


# ---------------------------------------------------------------------------
# selective scan with N state entries per channel
# ---------------------------------------------------------------------------


def sscan_ckpt_bytes(B: int, T: int, D: int, N: int) -> int:
    return int(_lib.lib().cla_sscan_ckpt_bytes(B, T, D, N))


def sscan_workspace_bytes(B: int, T: int, D: int, N: int, backward: bool = True,
                          have_ckpt: bool = True) -> int:
    return int(_lib.lib().cla_sscan_workspace_bytes(B, T, D, N, 1 if backward else 0,
                                                    1 if have_ckpt else 0))


def selective_scan(x, delta, A, Bm, Cm, h0=None, *, want_final=True, save_ckpt=False):
    """h_t[d,n] = exp(delta_t[d] A[d,n]) h_{t-1}[d,n] + delta_t[d] B_t[n] x_t[d],
    y_t[d] = sum_n C_t[n] h_t[d,n].  x, delta: [B, T, D] fp32; A: [D, N];
    Bm, Cm: [B, T, N]; h0: [B, D, N] or None.  Returns (y, h_T or None) and,
    with save_ckpt, the checkpoints for ``selective_scan_bwd`` as a third item."""
    B, T, D = x.shape
    N = A.shape[1]
    dev = x.device
    _need(x, "x", torch.float32, (B, T, D), dev)
    _need(delta, "delta", torch.float32, (B, T, D), dev)
    _need(A, "A", torch.float32, (D, N), dev)
    _need(Bm, "Bm", torch.float32, (B, T, N), dev)
    _need(Cm, "Cm", torch.float32, (B, T, N), dev)
    _opt(h0, "h0", torch.float32, (B, D, N), dev)
    y = torch.empty((B, T, D), dtype=torch.float32, device=dev)
    hT = torch.empty((B, D, N), dtype=torch.float32, device=dev) if want_final else None
    L = _lib.lib()
    ck = None
    if save_ckpt:
        nb = int(L.cla_sscan_ckpt_bytes(B, T, D, N))
        ck = torch.empty(max(nb // 4, 1), dtype=torch.float32, device=dev)
    ws, wsb = _workspace(int(L.cla_sscan_workspace_bytes(B, T, D, N, 0, 0)), dev)
    st = L.cla_sscan_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(h0), _ptr(y),
                         _ptr(hT), _ptr(ck), B, T, D, N, _ptr(ws), wsb, _stream(dev))
    _lib.check("cla_sscan_fwd", st)
    return (y, hT, ck) if save_ckpt else (y, hT)


def selective_scan_bwd(x, delta, A, Bm, Cm, h0, dy, dhT=None, *, ckpt=None, want_dh0=True,
                       workspace=None):
    """Backward of ``selective_scan``: returns (dx, ddelta, dA, dB, dC, dh0).
    ``ckpt`` is the forward's checkpoints (save_ckpt=True) or None (the call
    then recomputes them)."""
    B, T, D = x.shape
    N = A.shape[1]
    dev = x.device
    _need(x, "x", torch.float32, (B, T, D), dev)
    _need(delta, "delta", torch.float32, (B, T, D), dev)
    _need(A, "A", torch.float32, (D, N), dev)
    _need(Bm, "Bm", torch.float32, (B, T, N), dev)
    _need(Cm, "Cm", torch.float32, (B, T, N), dev)
    _opt(h0, "h0", torch.float32, (B, D, N), dev)
    _need(dy, "dy", torch.float32, (B, T, D), dev)
    _opt(dhT, "dhT", torch.float32, (B, D, N), dev)
    dx = torch.empty_like(x)
    dd = torch.empty_like(delta)
    dA = torch.empty((D, N), dtype=torch.float32, device=dev)
    dB = torch.empty((B, T, N), dtype=torch.float32, device=dev)
    dC = torch.empty((B, T, N), dtype=torch.float32, device=dev)
    dh0 = torch.empty((B, D, N), dtype=torch.float32, device=dev) if want_dh0 else None
    L = _lib.lib()
    nbytes = int(L.cla_sscan_workspace_bytes(B, T, D, N, 1, 0 if ckpt is None else 1))
    if workspace is None:
        ws, wsb = _workspace(nbytes, dev)
    else:
        ws, wsb = workspace, workspace.numel() * workspace.element_size()
    st = L.cla_sscan_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(h0), _ptr(ckpt),
                         _ptr(dy), _ptr(dhT), _ptr(dx), _ptr(dd), _ptr(dA), _ptr(dB), _ptr(dC),
                         _ptr(dh0), B, T, D, N, _ptr(ws), wsb, _stream(dev))
    _lib.check("cla_sscan_bwd", st)
    return dx, dd, dA, dB, dC, dh0
