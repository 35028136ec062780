"""MI355X-native gated linear-recurrence scans (libcla).

Python binding over the C ABI in include/cla.h.  Tensors are torch tensors on
a ROCm device; torch provides device memory and the current stream, and every
step of the computation runs in the library's HIP kernels.

    h, hT              = scan(a, b, h0=None)
    da, db, dh0        = scan_bwd(a, h, h0, dh, dhT=None)
    o, ST              = chunked_linear_attn(q, k, v, log_decay, S0=None)
    dq, dk, dv, dl, dS0 = chunked_linear_attn_bwd(q, k, v, log_decay, S0, dO, dST=None)

    # training: the forward keeps the states the backward's segments start from
    o, S_T, saved = chunked_linear_attn(q, k, v, log_decay, S0, save_states=True)
    dq, dk, dv, dl, dS0 = chunked_linear_attn_bwd(q, k, v, log_decay, S0, dO, saved=saved)

    # one log decay per key dimension (log_decay [B, H, T, DK])
    o, ST              = gla(q, k, v, log_decay, S0=None)
    dq, dk, dv, dl, dS0 = gla_bwd(q, k, v, log_decay, S0, dO, dST=None)

    # selective scan, N state entries per channel (fp32)
    y, hT, ckpt        = selective_scan(x, delta, A, Bm, Cm, h0=None, save_ckpt=True)
    dx, ddelta, dA, dB, dC, dh0 = selective_scan_bwd(x, delta, A, Bm, Cm, h0, dy, ckpt=ckpt)

    # decays the chunkwise calls do not accept (NaN, +inf; for gla also > 0
    # and -inf), counted on the device; set_input_checks(True) runs the check
    # at the start of chunked_linear_attn[_bwd] and gla[_bwd]
    check_log_decay(log_decay, kind="scalar" | "gla")

    # autograd: chunkwise_linear_attention_amd.autograd.{scan_fn,
    # chunked_linear_attn_fn, gla_fn, selective_scan_fn}
"""

from . import autograd  # noqa: F401
from ._lib import ClaError, lib  # noqa: F401
from .api import (  # noqa: F401
    check_log_decay,
    log_decay_counts,
    set_input_checks,
    chunked_linear_attn,
    chunked_linear_attn_bwd,
    scan,
    scan_bwd,
    scan_fwd_noalloc,
    scan_workspace_bytes,
    chunk_workspace_bytes,
    chunk_saved_bytes,
    gla,
    gla_bwd,
    gla_saved_bytes,
    gla_workspace_bytes,
    selective_scan,
    selective_scan_bwd,
    sscan_ckpt_bytes,
    sscan_workspace_bytes,
)

__all__ = ["scan", "scan_bwd", "scan_fwd_noalloc", "chunked_linear_attn", "chunked_linear_attn_bwd",
           "scan_workspace_bytes", "chunk_workspace_bytes", "chunk_saved_bytes", "gla", "gla_bwd", "gla_saved_bytes",
           "gla_workspace_bytes", "selective_scan", "selective_scan_bwd", "sscan_ckpt_bytes",
           "sscan_workspace_bytes", "check_log_decay", "log_decay_counts", "set_input_checks",
           "ClaError"]
