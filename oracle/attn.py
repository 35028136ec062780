"""Oracle for the matrix-state recurrence (gated linear attention) -- TEST
INFRASTRUCTURE ONLY.

For one head, with keys/queries of width dk and values of width dv:

    S_t = a_t S_{t-1} + k_t v_t^T          (S_t is dk x dv, rows by key)
    o_t = S_t^T q_t                          (update first, then read)
    a_t = exp(l_t)                           (l = log decay)

Every quantity is float64.  Per-head arrays have time first: q, k [T, dk],
v, o [T, dv], l [T], S [dk, dv].  Batched helpers take [B, H, T, ...].

Citations (page title, then section / equation):
  ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
  LA2 = "Lightning Attention-2: A Free Lunch for Handling Unlimited Sequence
        Lengths in Large Language Models" (paper-graph-ui summary)
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Forward, recurrent mode.  ZTF "Scans over vector and matrix states" (the
# linear-attention update) and "The chunkwise algorithm" (the recurrence with
# one scalar decay per step, S_0 the initial state); LA2 Eq. 4 for constant
# decay.
# ---------------------------------------------------------------------------


def la_loop(q, k, v, l, S0=None):
    """Per-token recurrence for one head.  Returns (o [T, dv], S_T [dk, dv])."""
    q, k, v, l = _f64(q), _f64(k), _f64(v), _f64(l)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((T, dv))
    for t in range(T):
        S = np.exp(l[t]) * S + np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def la_loop_states(q, k, v, l, S0=None):
    """All states S_0..S_T of the loop (tiny T only): [T + 1, dk, dv]."""
    q, k, v, l = _f64(q), _f64(k), _f64(v), _f64(l)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    out = np.empty((T + 1, dk, dv))
    out[0] = S
    for t in range(T):
        S = np.exp(l[t]) * S + np.outer(k[t], v[t])
        out[t + 1] = S
    return out


# ---------------------------------------------------------------------------
# Matrix mode.  ZTF "The chunkwise algorithm" (the sequence-mixing matrix):
# O = M V with M_ts = a_{t:s} q_t^T k_s for s <= t, a_{t:s} = a_t ... a_{s+1}
# (1 on the diagonal).  A nonzero S_0 reaches the read at t through
# a_{t:0} = a_t ... a_1 (ZTF "Scans over vector and matrix states": applying
# the prefixes to the initial state).  Segment products are built by
# multiplications only (ZTF "Long products without underflow").
# ---------------------------------------------------------------------------


def decay_matrix(l):
    """T x T lower-triangular a_{t:s} (0-based rows t and columns s; the
    product of a over steps s+1..t), diagonal 1."""
    a = np.exp(_f64(l))
    T = a.shape[0]
    M = np.zeros((T, T))
    for s in range(T):
        p = 1.0
        M[s, s] = 1.0
        for t in range(s + 1, T):
            p = p * a[t]
            M[t, s] = p
    return M


def prefix_decay(l):
    """a_{t:0} = a_t ... a_1 for t = 1..T (0-based index t-1)."""
    a = np.exp(_f64(l))
    out = np.empty_like(a)
    p = 1.0
    for t in range(a.shape[0]):
        p = p * a[t]
        out[t] = p
    return out


def la_matrix_mode(q, k, v, l, S0=None):
    """Brute-force quadratic form.  Returns (o, S_T)."""
    q, k, v, l = _f64(q), _f64(k), _f64(v), _f64(l)
    T, dk = q.shape
    dv = v.shape[1]
    M = decay_matrix(l)
    o = ((q @ k.T) * M) @ v
    # S_T = sum_s a_{T:s} k_s v_s^T (+ a_{T:0} S_0); row T-1 of M holds a_{T:s}
    ST = (k * M[T - 1][:, None]).T @ v if T > 0 else np.zeros((dk, dv))
    if S0 is not None:
        S0 = _f64(S0)
        P = prefix_decay(l)
        o = o + (q * P[:, None]) @ S0
        ST = ST + (P[T - 1] if T > 0 else 1.0) * S0
    return o, ST


# ---------------------------------------------------------------------------
# Chunkwise algorithm, in the order ZTF "The chunkwise algorithm" states it.
# Chunk j covers steps t0+1 .. t0+Tc (the last chunk may be shorter).  Three
# segment products:
#   mask     L_rs   = a_{t0+r : t0+s} for r >= s (diagonal 1), else 0
#   lambda_r        = a_{t0+r : t0}   (decay from the chunk start; includes
#                                      the first token's own decay)
#   gamma_s         = a_{t0+n : t0+s} (decay to the chunk end; excludes the
#                                      writing token's decay, so gamma_n = 1)
# and
#   O_[j] = (Q_[j] K_[j]^T (.) L) V_[j] + diag(lambda) Q_[j] S_[j-1]
#   S_[j] = a_{t0+n : t0} S_[j-1] + K_[j]^T diag(gamma) V_[j]
# LA2 Eq. 8 and Eq. 10 are the constant-decay case; LA2 prints
# Lambda = diag(lambda^0 .. lambda^{B-1}), which the option
# ``la2_printed_lambda`` reproduces (it gives the same outputs but a final
# state decayed once too often -- see the tests).
# ---------------------------------------------------------------------------


def la_chunkwise(q, k, v, l, S0=None, Tc=64, la2_printed_lambda=False):
    q, k, v, l = _f64(q), _f64(k), _f64(v), _f64(l)
    T, dk = q.shape
    dv = v.shape[1]
    a = np.exp(l)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((T, dv))
    for t0 in range(0, T, Tc):
        n = min(Tc, T - t0)
        aj = a[t0:t0 + n]
        Lm = decay_matrix(l[t0:t0 + n])
        lam = np.empty(n)
        p = 1.0
        for r in range(n):
            p = p * aj[r]
            lam[r] = p
        total = lam[n - 1]
        gam = np.empty(n)
        p = 1.0
        for s in range(n - 1, -1, -1):
            gam[s] = p
            p = p * aj[s]
        if la2_printed_lambda:
            # LA2's Lambda = diag(lambda^0 .. lambda^{B-1}) on the inter term
            # and lambda^B Lambda^{-1} = diag(lambda^B .. lambda^1) on the
            # update, for a constant decay lambda = a
            lam_c = aj[0]
            lam = lam_c ** np.arange(n)
            gam = lam_c ** (n - np.arange(n))
        Q, K, V = q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n]
        o[t0:t0 + n] = ((Q @ K.T) * Lm) @ V + (lam[:, None] * Q) @ S
        S = total * S + (K * gam[:, None]).T @ V
    return o, S


# ---------------------------------------------------------------------------
# Backward by the adjoint recurrence.  ZTF "The backward pass of linear
# attention": the read o_t = S_t^T q_t gives S_t the direct gradient
# q_t obar_t^T, so the adjoint obeys (reverse time, decays shifted one place,
# ZTF "The backward pass is a scan in reverse")
#     Sbar_T = q_T obar_T^T (+ dS_T, the gradient at the returned final state)
#     Sbar_t = q_t obar_t^T + a_{t+1} Sbar_{t+1}
# and each step has four gradients
#     qbar_t = S_t obar_t,  kbar_t = Sbar_t v_t,  vbar_t = Sbar_t^T k_t,
#     abar_t = <Sbar_t, S_{t-1}>   (so lbar_t = a_t abar_t),
# with dS_0 = a_1 Sbar_1.  This is the direct definition; it stores states.
# ---------------------------------------------------------------------------


def la_bwd_loop(q, k, v, l, S0, dO, dST=None):
    """Returns (dq [T,dk], dk [T,dk], dv [T,dv], dl [T], dS0 [dk,dv])."""
    q, k, v, l, dO = _f64(q), _f64(k), _f64(v), _f64(l), _f64(dO)
    T, dk = q.shape
    dv = v.shape[1]
    a = np.exp(l)
    Ss = la_loop_states(q, k, v, l, S0)  # Ss[t] = S_t, t = 0..T
    Sbar = np.zeros((dk, dv)) if dST is None else np.array(dST, dtype=np.float64)
    gq = np.empty((T, dk))
    gk = np.empty((T, dk))
    gv = np.empty((T, dv))
    gl = np.empty(T)
    for t in range(T - 1, -1, -1):  # 0-based t is step t+1
        if t < T - 1:
            Sbar = a[t + 1] * Sbar
        Sbar = Sbar + np.outer(q[t], dO[t])
        gq[t] = Ss[t + 1] @ dO[t]
        gk[t] = Sbar @ v[t]
        gv[t] = Sbar.T @ k[t]
        gl[t] = a[t] * np.sum(Sbar * Ss[t])
    dS0 = a[0] * Sbar if T > 0 else Sbar.copy()
    return gq, gk, gv, gl, dS0


def dlog_closed_form(q, k, dq, dk, ST=None, dST=None):
    """Decay gradient without states.  ZTF "The backward pass of linear
    attention" (closed form after Yang et al. 2023, Section 4.3):
        dl_u = sum_{t >= u} q_t . qbar_t - sum_{s >= u} k_s . kbar_s
    plus, when the final state is itself an output with gradient dS_T, the
    term <S_T, dS_T> on every u: every path into the final state crosses
    every step (reading of the page for a returned final state)."""
    q, k, dq, dk = _f64(q), _f64(k), _f64(dq), _f64(dk)
    r = np.sum(q * dq, axis=1) - np.sum(k * dk, axis=1)
    out = np.cumsum(r[::-1])[::-1].copy()
    if ST is not None and dST is not None:
        out = out + np.sum(_f64(ST) * _f64(dST))
    return out


# ---------------------------------------------------------------------------
# Batched wrappers over [B, H, T, ...].
# ---------------------------------------------------------------------------


def la_fwd_batched(q, k, v, l, S0=None, fn=la_loop):
    B, H, T, _ = q.shape
    dk, dv = q.shape[-1], v.shape[-1]
    o = np.empty((B, H, T, dv))
    ST = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            o[b, h], ST[b, h] = fn(q[b, h], k[b, h], v[b, h], l[b, h],
                                   None if S0 is None else S0[b, h])
    return o, ST


def la_bwd_batched(q, k, v, l, S0, dO, dST=None):
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dq = np.empty((B, H, T, dk))
    dkk = np.empty((B, H, T, dk))
    dvv = np.empty((B, H, T, dv))
    dl = np.empty((B, H, T))
    dS0 = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            dq[b, h], dkk[b, h], dvv[b, h], dl[b, h], dS0[b, h] = la_bwd_loop(
                q[b, h], k[b, h], v[b, h], l[b, h],
                None if S0 is None else S0[b, h], dO[b, h],
                None if dST is None else dST[b, h])
    return dq, dkk, dvv, dl, dS0
