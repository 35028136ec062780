"""Oracle for the selective scan with N state entries per channel (Mamba-1's
recurrence) -- TEST INFRASTRUCTURE ONLY.

For one sequence with D channels, each keeping N state numbers:

    a_t[d, n] = exp(delta_t[d] * A[d, n])          (decay, one per entry)
    b_t[d, n] = delta_t[d] * B_t[n] * x_t[d]       (the token written in)
    h_t[d, n] = a_t[d, n] h_{t-1}[d, n] + b_t[d, n]
    y_t[d]    = sum_n C_t[n] h_t[d, n]

ZTF "Parallel scan", section "Scans over vector and matrix states": in Mamba
every channel keeps N state numbers, each with its own decay, so the
transition is diagonal and b_t is the token's input written into the state.
Section "What limits a recurrent layer" (the paragraph on Mamba's kernel and on
Mamba-2's chunks) gives the decay for channel d and entry n as
exp(delta_{t,d} A_{d,n}), with a step size per channel and token and a learned
rate per channel and entry, and says the fused kernel contracts the state with
C inside the kernel and never writes the (batch, T, channels, N) state
tensor.  The backward is the reverse-time adjoint of section "The backward
pass is a scan in reverse", elementwise per (d, n), followed by the chain rule
through the discretization above.

Every quantity is float64.  Per-sequence arrays have time first: x, delta, y
[T, D]; B, C [T, N]; A [D, N]; h0, hT [D, N].  Batched helpers add a leading
batch axis to everything but A.

Citations (page title, then section):
  ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def discretize(x, delta, A, Bm):
    """Per-token decays and inputs of the N-entry diagonal recurrence:
    a[t, d, n] = exp(delta[t, d] A[d, n]), b[t, d, n] = delta[t, d] B[t, n]
    x[t, d] (ZTF "What limits a recurrent layer", Mamba-1's decay; "Scans over
    vector and matrix states", b_t = the token's input written into the
    state)."""
    x, delta, A, Bm = (_f64(v) for v in (x, delta, A, Bm))
    a = np.exp(delta[:, :, None] * A[None, :, :])
    b = (delta * x)[:, :, None] * Bm[:, None, :]
    return a, b


def sscan_states(x, delta, A, Bm, h0=None):
    """All states h_1..h_T [T, D, N] by the sequential loop (each step applies
    the pair (a_t, b_t) to the previous state)."""
    a, b = discretize(x, delta, A, Bm)
    T, D, N = a.shape
    h = np.zeros((D, N)) if h0 is None else _f64(h0).copy()
    out = np.empty((T, D, N))
    for t in range(T):
        h = a[t] * h + b[t]
        out[t] = h
    return out


def sscan_loop(x, delta, A, Bm, Cm, h0=None):
    """Forward: y [T, D] with y_t[d] = sum_n C_t[n] h_t[d, n], and h_T [D, N]."""
    x, delta, A, Bm, Cm = (_f64(v) for v in (x, delta, A, Bm, Cm))
    T, D = x.shape
    N = A.shape[1]
    if T == 0:
        return np.zeros((0, D)), (np.zeros((D, N)) if h0 is None else _f64(h0).copy())
    hs = sscan_states(x, delta, A, Bm, h0)
    y = np.einsum("tdn,tn->td", hs, Cm)
    return y, hs[-1].copy()


def sscan_matrix_mode(x, delta, A, Bm, Cm, h0=None):
    """The same outputs written out as sums over paths, with no recurrence:
    h_t[d, n] = exp(A[d, n] sum_{r<=t} delta_r[d]) h0[d, n]
              + sum_{s<=t} exp(A[d, n] sum_{s<r<=t} delta_r[d]) b_s[d, n],
    each product of decays a_{t:s} taken as one exponential of a summed step
    size (the decay of several steps of one entry is the exponential of A
    times the summed deltas).  O(T^2 D N): tiny inputs only."""
    x, delta, A, Bm, Cm = (_f64(v) for v in (x, delta, A, Bm, Cm))
    T, D = x.shape
    N = A.shape[1]
    b = (delta * x)[:, :, None] * Bm[:, None, :]
    y = np.zeros((T, D))
    hT = np.zeros((D, N)) if h0 is None else _f64(h0).copy()
    for t in range(T):
        h = np.zeros((D, N))
        if h0 is not None:
            h += np.exp(A * delta[: t + 1].sum(axis=0)[:, None]) * _f64(h0)
        for s in range(t + 1):
            span = delta[s + 1: t + 1].sum(axis=0)          # steps s+1..t
            h += np.exp(A * span[:, None]) * b[s]
        y[t] = h @ Cm[t]
        hT = h
    return y, hT


def sscan_bwd_loop(x, delta, A, Bm, Cm, h0, dy, dhT=None):
    """Backward of ``sscan_loop``.  Returns (dx [T, D], ddelta [T, D], dA [D, N],
    dB [T, N], dC [T, N], dh0 [D, N]).

    Adjoint (ZTF "The backward pass is a scan in reverse", per entry):
        hbar_T = g_T (+ dh_T),  hbar_t = g_t + a_{t+1} hbar_{t+1},
        g_t[d, n] = C_t[n] dy_t[d]  (y_t reads h_t through C_t),
        dL/da_t = hbar_t h_{t-1},  dL/db_t = hbar_t,  dh0 = a_1 hbar_1.
    Chain rule through a = exp(delta A) and b = delta B x:
        ddelta_t[d] = sum_n (dL/da_t a_t A)[d, n] + sum_n hbar_t[d, n] B_t[n] x_t[d]
        dA[d, n]    = sum_t dL/da_t[d, n] a_t[d, n] delta_t[d]
        dx_t[d]     = delta_t[d] sum_n hbar_t[d, n] B_t[n]
        dB_t[n]     = sum_d hbar_t[d, n] delta_t[d] x_t[d]
        dC_t[n]     = sum_d dy_t[d] h_t[d, n]
    """
    x, delta, A, Bm, Cm, dy = (_f64(v) for v in (x, delta, A, Bm, Cm, dy))
    T, D = x.shape
    N = A.shape[1]
    h0f = np.zeros((D, N)) if h0 is None else _f64(h0)
    if T == 0:
        dh0 = np.zeros((D, N)) if dhT is None else _f64(dhT).copy()
        return (np.zeros((0, D)), np.zeros((0, D)), np.zeros((D, N)), np.zeros((0, N)),
                np.zeros((0, N)), dh0)
    a, _ = discretize(x, delta, A, Bm)
    hs = sscan_states(x, delta, A, Bm, h0f)
    prev = np.concatenate([h0f[None], hs[:-1]], axis=0)     # h_{t-1}
    hbar = np.zeros((D, N)) if dhT is None else _f64(dhT).copy()
    dx = np.zeros((T, D))
    ddelta = np.zeros((T, D))
    dA = np.zeros((D, N))
    dB = np.zeros((T, N))
    dC = np.einsum("td,tdn->tn", dy, hs)
    for t in range(T - 1, -1, -1):
        if t + 1 < T:
            hbar = a[t + 1] * hbar
        hbar = hbar + dy[t][:, None] * Cm[t][None, :]
        da = hbar * prev[t]
        ddelta[t] = (da * a[t] * A).sum(axis=1) + (hbar * Bm[t][None, :]).sum(axis=1) * x[t]
        dA += da * a[t] * delta[t][:, None]
        dx[t] = delta[t] * (hbar * Bm[t][None, :]).sum(axis=1)
        dB[t] = (hbar * (delta[t] * x[t])[:, None]).sum(axis=0)
    dh0 = a[0] * hbar
    return dx, ddelta, dA, dB, dC, dh0


def sscan_fwd_batched(x, delta, A, Bm, Cm, h0=None):
    """[Bt, T, D] inputs (B, C [Bt, T, N], h0 [Bt, D, N] or None): (y, hT)."""
    x = _f64(x)
    Bt, T, D = x.shape
    N = np.asarray(A).shape[1]
    y = np.empty((Bt, T, D))
    hT = np.empty((Bt, D, N))
    for i in range(Bt):
        y[i], hT[i] = sscan_loop(x[i], delta[i], A, Bm[i], Cm[i],
                                 None if h0 is None else h0[i])
    return y, hT


def sscan_bwd_batched(x, delta, A, Bm, Cm, h0, dy, dhT=None):
    """Batched backward; dA is summed over the batch (A is shared)."""
    x = _f64(x)
    Bt, T, D = x.shape
    N = np.asarray(A).shape[1]
    dx = np.empty((Bt, T, D))
    dd = np.empty((Bt, T, D))
    dA = np.zeros((D, N))
    dB = np.empty((Bt, T, N))
    dC = np.empty((Bt, T, N))
    dh0 = np.empty((Bt, D, N))
    for i in range(Bt):
        r = sscan_bwd_loop(x[i], delta[i], A, Bm[i], Cm[i], None if h0 is None else h0[i],
                           dy[i], None if dhT is None else dhT[i])
        dx[i], dd[i], dAi, dB[i], dC[i], dh0[i] = r
        dA += dAi
    return dx, dd, dA, dB, dC, dh0
