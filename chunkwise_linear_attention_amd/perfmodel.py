"""Algorithmic work of the hot path: bytes and FLOPs per unit, and rooflines.

These are the counts the throughput and roofline figures are priced against.
They count what the method itself must move or compute, not what a given
kernel happens to move.

Citations (page title, then section):
  ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
"""

from __future__ import annotations

import math

# MI355X published peaks (dense; no sparsity).
PEAK_HBM_GBS = 8000.0          # GB/s
PEAK_BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3  # fp32 vector


# --------------------------------------------------------------------------
# chunk-size arithmetic: ZTF "How big should a chunk be"
# --------------------------------------------------------------------------


def chunk_flops(Tc: int, dk: int, dv: int) -> int:
    """Matrix-product FLOPs of one full chunk of the forward: intra scores
    2 Tc^2 dk, their product with V 2 Tc^2 dv, inter read 2 Tc dk dv, state
    update 2 Tc dk dv (an m x k by k x n product costs 2 m k n)."""
    return 2 * Tc * Tc * dk + 2 * Tc * Tc * dv + 4 * Tc * dk * dv


def sequence_flops(T: int, Tc: int, dk: int, dv: int) -> int:
    """Forward FLOPs over a sequence of T tokens in ceil(T / Tc) chunks (the
    last one shorter)."""
    full, rem = divmod(T, Tc)
    return full * chunk_flops(Tc, dk, dv) + (chunk_flops(rem, dk, dv) if rem else 0)


def balance_chunk(dk: int, dv: int) -> float:
    """Chunk length at which the quadratic and linear parts cost the same:
    2 Tc^2 (dk + dv) = 4 Tc dk dv  ->  Tc* = 2 dk dv / (dk + dv)."""
    return 2.0 * dk * dv / (dk + dv)


def onchip_bytes(Tc: int, d: int) -> dict:
    """Bytes one chunk keeps on chip: bf16 Q, K, V; fp32 scores; fp32 state."""
    return {"inputs_bf16": 3 * Tc * d * 2, "scores_f32": Tc * Tc * 4,
            "state_f32": d * d * 4}


# --------------------------------------------------------------------------
# per-unit algorithmic bytes / FLOPs of the two regimes
# --------------------------------------------------------------------------


def scan_bytes_per_elem(direction: str = "fwdbwd") -> int:
    """Diagonal scan, fp32: forward reads a, b and writes h (12 B); backward
    reads a, h, dh and writes da, db (20 B)."""
    return {"fwd": 12, "bwd": 20, "fwdbwd": 32}[direction]


def chunk_bytes_per_token_head(dk: int, dv: int, direction: str = "fwdbwd") -> int:
    """Chunkwise, bf16 I/O, fp32 log decay: forward reads q, k, v, l and
    writes o; backward reads q, k, v, dO, l and writes dq, dk, dv, dl."""
    fwd = 2 * dk + 2 * dk + 2 * dv + 4 + 2 * dv
    bwd = 2 * dk * 2 + 2 * dv + 2 * dv + 4 + 2 * dk * 2 + 2 * dv + 4
    return {"fwd": fwd, "bwd": bwd, "fwdbwd": fwd + bwd}[direction]


def chunk_state_bytes(dk: int, dv: int) -> int:
    """One fp32 dk x dv state (S0, S_T, dS_T or dS0) per (batch, head)."""
    return 4 * dk * dv


def chunk_flops_per_token_head(Tc: int, dk: int, dv: int, direction: str = "fwdbwd") -> int:
    """Forward 2 Tc (dk + dv) + 4 dk dv; backward 2 Tc (3 dk + 2 dv) + 10 dk dv
    (dQ pass with the chunk-state recompute, dK/dV pass with the adjoint
    state update).  Masked upper triangles are counted as computed."""
    fwd = 2 * Tc * (dk + dv) + 4 * dk * dv
    bwd = 2 * Tc * (3 * dk + 2 * dv) + 10 * dk * dv
    return {"fwd": fwd, "bwd": bwd, "fwdbwd": fwd + bwd}[direction]


def roofline_seconds(bytes_: float, flops: float = 0.0,
                     peak_gbs: float = PEAK_HBM_GBS,
                     peak_tflops: float = PEAK_BF16_TFLOPS) -> float:
    return max(bytes_ / (peak_gbs * 1e9), flops / (peak_tflops * 1e12))


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def log2ceil(n: int) -> int:
    return max(0, math.ceil(math.log2(n))) if n > 0 else 0


# --------------------------------------------------------------------------
# per-kernel algorithmic bytes of the chunkwise implementation (per
# token-head unless stated): what each kernel itself must read and write
# --------------------------------------------------------------------------


def chunk_kernel_bytes(name: str, dk: int, dv: int) -> int:
    """chunk_fwd : q, k, v, l in; o out (the forward per-unit figure).
    chunk_dq    : dO, v, k, l, q in; dq, q.dq out (plus, with segments, one
                  fp32 state per segment, not per token).
    chunk_dkdv  : q, k, v, dO, l, q.dq in; dk, dv, dl out (the decay
                  gradient's suffix sums are formed in this pass).
    *_segments  : the inputs of the state recurrence only (k, v, l)."""
    table = {
        "chunk_fwd": chunk_bytes_per_token_head(dk, dv, "fwd"),
        "chunk_dq": 2 * dv + 2 * dv + 2 * dk + 4 + 2 * dk + 2 * dk + 4,
        "chunk_dkdv": 2 * dk + 2 * dk + 2 * dv + 2 * dv + 4 + 4 + 2 * dk + 2 * dv + 4,
        "chunk_fwd_segments": 2 * dk + 2 * dv + 4,
        "chunk_dq_segments": 2 * dv + 2 * dk + 4,
    }
    return table[name]


# --------------------------------------------------------------------------
# one decay per key dimension (gated linear attention): l is [.., T, dk] fp32
# --------------------------------------------------------------------------


def gla_bytes_per_token_head(dk: int, dv: int, direction: str = "fwdbwd") -> int:
    """Forward reads q, k, v and the dk log decays and writes o; backward
    reads q, k, v, dO, l and writes dq, dk, dv and the dk decay gradients."""
    fwd = 2 * dk + 2 * dk + 2 * dv + 4 * dk + 2 * dv
    bwd = (2 * dk + 2 * dk + 2 * dv + 2 * dv + 4 * dk) + (2 * dk + 2 * dk + 2 * dv + 4 * dk)
    return {"fwd": fwd, "bwd": bwd, "fwdbwd": fwd + bwd}[direction]


def gla_flops_per_token_head(Tc: int, dk: int, dv: int, direction: str = "fwdbwd") -> int:
    """The same products as the scalar-decay chunkwise form (the decay enters
    as scaling of the operands, which is not counted)."""
    return chunk_flops_per_token_head(Tc, dk, dv, direction)


def gla_kernel_bytes(name: str, dk: int, dv: int) -> int:
    """gla_fwd  : q, k, v, l in; o out.
    gla_dq   : q, k, v, dO, l in; dq and the fp32 products q.dq out (plus one
               fp32 state per segment of 16 chunks, not per token).
    gla_dkdv : q, k, v, dO, l, q.dq in; dk, dv, dl out."""
    table = {
        "gla_fwd": gla_bytes_per_token_head(dk, dv, "fwd"),
        "gla_dq": 2 * dk + 2 * dk + 2 * dv + 2 * dv + 4 * dk + 2 * dk + 4 * dk,
        "gla_dkdv": 2 * dk + 2 * dk + 2 * dv + 2 * dv + 4 * dk + 4 * dk + 2 * dk + 2 * dv + 4 * dk,
    }
    return table[name]


# --------------------------------------------------------------------------
# selective scan with N state entries per channel: bound by VALU issue
# --------------------------------------------------------------------------

# One fp32 VALU operation per lane per cycle: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz.  (The 157.3 TFLOP/s fp32 figure counts an FMA as 2 flops and
# packed two-wide math; the kernels here issue unpacked ops.)
PEAK_VALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12   # 39.32 T lane-ops/s
EXP_SLOTS = 4                                   # v_exp_f32 issues at quarter rate


def sscan_bytes(B: int, T: int, D: int, N: int, direction: str = "fwdbwd") -> int:
    """Forward reads x, delta (per token and channel), B, C (per token), A,
    and writes y; backward reads x, delta, dy, B, C, A and writes dx, ddelta,
    dB, dC, dA.  The [B, T, D, N] states are never moved."""
    fwd = B * T * (4 * D * 3 + 4 * N * 2) + 4 * D * N
    bwd = B * T * (4 * D * 5 + 4 * N * 4) + 4 * D * N * 2
    return {"fwd": fwd, "bwd": bwd, "fwdbwd": fwd + bwd}[direction]


def sscan_ops_per_element(direction: str = "fwdbwd") -> int:
    """VALU lane-operations per (token, channel, entry), an exp counted as
    EXP_SLOTS.  Forward: delta*A, exp, (delta x)*B, the state FMA, the output
    FMA.  Backward: the state recomputed (4 ops and an exp), the decay again
    (1 op and an exp), the adjoint FMA and C*dy, dL/da*a (2), the delta and A
    gradients (2 FMAs), the B sum, and the dB and dC terms (2)."""
    fwd = 4 + EXP_SLOTS
    bwd = (3 + EXP_SLOTS) + (1 + EXP_SLOTS) + 2 + 2 + 2 + 1 + 2
    return {"fwd": fwd, "bwd": bwd, "fwdbwd": fwd + bwd}[direction]
