"""torch.autograd wrappers over the library's forward/backward pairs.

Each Function's forward calls the C-ABI forward and keeps what the matching
backward call takes (the inputs, plus the forward's saved segment states or
checkpoints where the library offers them); its backward calls the C-ABI
backward.  No arithmetic of the method runs here.  A gradient that arrives as
None (an output not used in the loss) is passed to the library as "absent"
(the final-state gradients) or as zeros (the per-token outputs).

    h, hT = scan_fn(a, b, h0)
    o, ST = chunked_linear_attn_fn(q, k, v, log_decay, S0)
    o, ST = gla_fn(q, k, v, log_decay, S0)
    y, hT = selective_scan_fn(x, delta, A, Bm, Cm, h0)
"""

from __future__ import annotations

import torch

from . import api


def _zeros_if_none(g, like):
    return torch.zeros_like(like) if g is None else g.contiguous()


class ScanFn(torch.autograd.Function):
    """h_t = a_t h_{t-1} + b_t (cla_scan_fwd / cla_scan_bwd)."""

    @staticmethod
    def forward(ctx, a, b, h0):
        h, hT = api.scan(a, b, h0)
        ctx.save_for_backward(a, h, h0)
        ctx.has_h0 = h0 is not None
        return h, hT

    @staticmethod
    def backward(ctx, dh, dhT):
        a, h, h0 = ctx.saved_tensors
        da, db, dh0 = api.scan_bwd(a, h, h0, _zeros_if_none(dh, h),
                                   None if dhT is None else dhT.contiguous(),
                                   want_dh0=ctx.has_h0)
        return da, db, dh0


class ChunkedLinearAttnFn(torch.autograd.Function):
    """S_t = exp(l_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, chunkwise
    (cla_chunk_fwd_saved / cla_chunk_bwd_saved)."""

    @staticmethod
    def forward(ctx, q, k, v, log_decay, S0):
        o, ST, saved = api.chunked_linear_attn(q, k, v, log_decay, S0, save_states=True)
        ctx.save_for_backward(q, k, v, log_decay, S0, saved)
        ctx.has_S0 = S0 is not None
        return o, ST

    @staticmethod
    def backward(ctx, dO, dST):
        q, k, v, l, S0, saved = ctx.saved_tensors
        dq, dk, dv, dl, dS0 = api.chunked_linear_attn_bwd(
            q, k, v, l, S0, _zeros_if_none(dO, v), None if dST is None else dST.contiguous(),
            want_dS0=ctx.has_S0, saved=saved)
        return dq, dk, dv, dl, dS0


class GLAFn(torch.autograd.Function):
    """The same with one decay per key dimension (cla_gla_fwd_saved /
    cla_gla_bwd_saved)."""

    @staticmethod
    def forward(ctx, q, k, v, log_decay, S0):
        o, ST, saved = api.gla(q, k, v, log_decay, S0, save_states=True)
        ctx.save_for_backward(q, k, v, log_decay, S0, saved)
        ctx.has_S0 = S0 is not None
        return o, ST

    @staticmethod
    def backward(ctx, dO, dST):
        q, k, v, l, S0, saved = ctx.saved_tensors
        dq, dk, dv, dl, dS0 = api.gla_bwd(q, k, v, l, S0, _zeros_if_none(dO, v),
                                          None if dST is None else dST.contiguous(),
                                          want_dS0=ctx.has_S0, saved=saved)
        return dq, dk, dv, dl, dS0


class SelectiveScanFn(torch.autograd.Function):
    """Selective scan with N state entries per channel (cla_sscan_fwd with
    checkpoints / cla_sscan_bwd)."""

    @staticmethod
    def forward(ctx, x, delta, A, Bm, Cm, h0):
        y, hT, ckpt = api.selective_scan(x, delta, A, Bm, Cm, h0, save_ckpt=True)
        ctx.save_for_backward(x, delta, A, Bm, Cm, h0, ckpt)
        ctx.has_h0 = h0 is not None
        return y, hT

    @staticmethod
    def backward(ctx, dy, dhT):
        x, delta, A, Bm, Cm, h0, ckpt = ctx.saved_tensors
        dx, dd, dA, dB, dC, dh0 = api.selective_scan_bwd(
            x, delta, A, Bm, Cm, h0, _zeros_if_none(dy, x),
            None if dhT is None else dhT.contiguous(), ckpt=ckpt, want_dh0=ctx.has_h0)
        return dx, dd, dA, dB, dC, dh0


def scan_fn(a, b, h0=None):
    return ScanFn.apply(a, b, h0)


def chunked_linear_attn_fn(q, k, v, log_decay, S0=None):
    return ChunkedLinearAttnFn.apply(q, k, v, log_decay, S0)


def gla_fn(q, k, v, log_decay, S0=None):
    return GLAFn.apply(q, k, v, log_decay, S0)


def selective_scan_fn(x, delta, A, Bm, Cm, h0=None):
    return SelectiveScanFn.apply(x, delta, A, Bm, Cm, h0)
