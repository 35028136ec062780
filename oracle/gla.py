"""Oracle for the matrix-state recurrence with one decay per key dimension
(gated linear attention) -- TEST INFRASTRUCTURE ONLY.

For one head, with keys/queries of width dk and values of width dv:

    S_t = diag(a_t) S_{t-1} + k_t v_t^T     (S_t is dk x dv, rows by key)
    o_t = S_t^T q_t                          (update first, then read)
    a_t = exp(l_t),  l_t in R^dk             (one log decay per key dimension)

ZTF "Parallel scan" lists the diagonal transition, one decay per state entry,
as the form gated linear attention uses (section "Scans over vector and
matrix states"), and states the GLA paper's recurrence S_t = G_t (.) S_{t-1}
+ k_t^T v_t in the same layout as the scalar one (section "The chunkwise
algorithm"): G_t holds a_t[d] in every column of row d.

Every quantity is float64.  Per-head arrays have time first: q, k [T, dk],
v, o [T, dv], l [T, dk], S [dk, dv].

Citations (page title, then section):
  ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Forward, recurrent mode (ZTF "The chunkwise algorithm", the GLA form of the
# recurrence; update first, then read).
# ---------------------------------------------------------------------------


def gla_loop(q, k, v, l, S0=None):
    """Per-token recurrence for one head.  Returns (o [T, dv], S_T [dk, dv])."""
    q, k, v, l = _f64(q), _f64(k), _f64(v), _f64(l)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((T, dv))
    for t in range(T):
        S = np.exp(l[t])[:, None] * S + np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def gla_loop_states(q, k, v, l, S0=None):
    """All states S_0..S_T of the loop: [T + 1, dk, dv]."""
    q, k, v, l = _f64(q), _f64(k), _f64(v), _f64(l)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    out = np.empty((T + 1, dk, dv))
    out[0] = S
    for t in range(T):
        S = np.exp(l[t])[:, None] * S + np.outer(k[t], v[t])
        out[t + 1] = S
    return out


# ---------------------------------------------------------------------------
# Matrix mode (ZTF "The chunkwise algorithm", the sequence-mixing matrix):
# with a vector decay the entry of the mixing matrix keeps the key dimension,
#     o_t = sum_{s <= t} (sum_d q_t[d] k_s[d] a_{t:s}[d]) v_s
#           + sum_d q_t[d] a_{t:0}[d] S_0[d, :],
# a_{t:s}[d] = a_t[d] ... a_{s+1}[d] (1 for s = t), built by multiplications
# only (ZTF "Long products without underflow").
# ---------------------------------------------------------------------------


def segment_products(l):
    """[T, T, dk]: entry (t, s, d) = a_{t:s}[d] for s <= t, else 0."""
    a = np.exp(_f64(l))
    T, dk = a.shape
    M = np.zeros((T, T, dk))
    for s in range(T):
        p = np.ones(dk)
        M[s, s] = p
        for t in range(s + 1, T):
            p = p * a[t]
            M[t, s] = p
    return M


def gla_matrix_mode(q, k, v, l, S0=None):
    """Brute-force quadratic form (tiny T).  Returns (o, S_T)."""
    q, k, v, l = _f64(q), _f64(k), _f64(v), _f64(l)
    T, dk = q.shape
    dv = v.shape[1]
    M = segment_products(l)                       # [t, s, d]
    W = np.einsum("td,sd,tsd->ts", q, k, M)       # the mixing matrix
    o = W @ v
    ST = np.zeros((dk, dv))
    if T > 0:
        ST = (k * M[T - 1]).T @ v                 # sum_s a_{T:s} k_s v_s^T
    if S0 is not None:
        S0 = _f64(S0)
        P = np.ones(dk)
        pre = np.empty((T, dk))
        a = np.exp(l)
        for t in range(T):
            P = P * a[t]
            pre[t] = P                            # a_{t:0}
        o = o + (q * pre) @ S0
        ST = ST + (pre[T - 1] if T > 0 else np.ones(dk))[:, None] * S0
    return o, ST


# ---------------------------------------------------------------------------
# Chunkwise algorithm (ZTF "The chunkwise algorithm") with the three segment
# products kept per key dimension:
#   mask     L[r, s, d] = a_{t0+r : t0+s}[d]  for r >= s (1 on the diagonal)
#   lambda_r[d]         = a_{t0+r : t0}[d]    (decay from the chunk start)
#   gamma_s[d]          = a_{t0+n : t0+s}[d]  (decay to the chunk end)
#   O_[j] = A V_[j] + (lambda (.) Q_[j]) S_[j-1],
#           A[r, s] = sum_d Q[r, d] K[s, d] L[r, s, d]
#   S_[j] = diag(a_{t0+n : t0}) S_[j-1] + (gamma (.) K_[j])^T V_[j]
# ---------------------------------------------------------------------------


def gla_chunkwise(q, k, v, l, S0=None, Tc=64):
    q, k, v, l = _f64(q), _f64(k), _f64(v), _f64(l)
    T, dk = q.shape
    dv = v.shape[1]
    a = np.exp(l)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((T, dv))
    for t0 in range(0, T, Tc):
        n = min(Tc, T - t0)
        aj = a[t0:t0 + n]
        L = segment_products(l[t0:t0 + n])
        lam = np.empty((n, dk))
        p = np.ones(dk)
        for r in range(n):
            p = p * aj[r]
            lam[r] = p
        gam = np.empty((n, dk))
        p = np.ones(dk)
        for s in range(n - 1, -1, -1):
            gam[s] = p
            p = p * aj[s]
        Q, K, V = q[t0:t0 + n], k[t0:t0 + n], v[t0:t0 + n]
        A = np.einsum("rd,sd,rsd->rs", Q, K, L)
        o[t0:t0 + n] = A @ V + (lam * Q) @ S
        S = lam[n - 1][:, None] * S + (K * gam).T @ V
    return o, S


# ---------------------------------------------------------------------------
# Backward by the adjoint recurrence (ZTF "The backward pass of linear
# attention", with the scalar decay replaced by the diagonal one: the state's
# row d decays by a_t[d]).  The read o_t = S_t^T q_t gives S_t the direct
# gradient q_t obar_t^T, so
#     Sbar_T = q_T obar_T^T (+ dS_T)
#     Sbar_t = q_t obar_t^T + diag(a_{t+1}) Sbar_{t+1}
#     qbar_t = S_t obar_t,  kbar_t = Sbar_t v_t,  vbar_t = Sbar_t^T k_t,
#     abar_t[d] = <Sbar_t[d, :], S_{t-1}[d, :]>,  lbar_t[d] = a_t[d] abar_t[d]
# and dS_0 = diag(a_1) Sbar_1.  This is the direct definition; it stores states.
# ---------------------------------------------------------------------------


def gla_bwd_loop(q, k, v, l, S0, dO, dST=None):
    """Returns (dq [T,dk], dk [T,dk], dv [T,dv], dl [T,dk], dS0 [dk,dv])."""
    q, k, v, l, dO = _f64(q), _f64(k), _f64(v), _f64(l), _f64(dO)
    T, dk = q.shape
    dv = v.shape[1]
    a = np.exp(l)
    Ss = gla_loop_states(q, k, v, l, S0)
    Sbar = np.zeros((dk, dv)) if dST is None else np.array(dST, dtype=np.float64)
    gq = np.empty((T, dk))
    gk = np.empty((T, dk))
    gv = np.empty((T, dv))
    gl = np.empty((T, dk))
    for t in range(T - 1, -1, -1):  # 0-based t is step t+1
        if t < T - 1:
            Sbar = a[t + 1][:, None] * Sbar
        Sbar = Sbar + np.outer(q[t], dO[t])
        gq[t] = Ss[t + 1] @ dO[t]
        gk[t] = Sbar @ v[t]
        gv[t] = Sbar.T @ k[t]
        gl[t] = a[t] * np.sum(Sbar * Ss[t], axis=1)
    dS0 = a[0][:, None] * Sbar if T > 0 else Sbar.copy()
    return gq, gk, gv, gl, dS0


def gla_dlog_closed_form(q, k, dq, dk, ST=None, dST=None):
    """Vector decay gradient without states (ZTF "The backward pass of linear
    attention": the closed form of Yang et al. 2023, Section 4.3, for a vector
    of decays per step).  The path argument runs per key dimension: raising
    l_u[d] scales exactly the contributions that cross step u through row d
    of the state, so
        dl_u[d] = sum_{t >= u} q_t[d] qbar_t[d] - sum_{s >= u} k_s[d] kbar_s[d]
    plus <S_T[d, :], dS_T[d, :]> on every u when the final state has a
    gradient (every path into it crosses every step)."""
    q, k, dq, dk = _f64(q), _f64(k), _f64(dq), _f64(dk)
    r = q * dq - k * dk                            # [T, dk]
    out = np.cumsum(r[::-1], axis=0)[::-1].copy()
    if ST is not None and dST is not None:
        out = out + np.sum(_f64(ST) * _f64(dST), axis=1)[None, :]
    return out
