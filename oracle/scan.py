"""Oracle for the diagonal linear recurrence -- TEST INFRASTRUCTURE ONLY.

    h_t = a_t * h_{t-1} + b_t,  t = 1..T,  h_0 given (zero unless stated)

Every quantity is float64.  Arrays are laid out [B, T, D] (channels last), the
layout the WIKI page's ``scan(a, b)`` uses ("over dim 1"), so that the time
axis is axis 1.  One-dimensional helpers take the time axis first.

Citations (page title, then section):
  ZTF  = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan)
  WIKI = "Parallel Scan" (aiwiki.thehackersbrain.dev)
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# The pair algebra.  ZTF "The scan for one number of state": applying step
# (a1, b1) and then (a2, b2) is the single step (a1 a2, a2 b1 + b2); the step
# that changes nothing is (1, 0).  The EARLIER step is the left argument.
# ---------------------------------------------------------------------------

IDENTITY = (1.0, 0.0)


def compose(p1, p2):
    """Return the pair for "p1, then p2" (p1 is the earlier step)."""
    a1, b1 = p1
    a2, b2 = p2
    return (a1 * a2, a2 * b1 + b2)


def compose_dense(p1, p2):
    """Matrix-affine steps (A, b): "p1, then p2".

    ZTF "Scans over vector and matrix states": the later step's matrix stands
    on the left in both components, (A2 A1, A2 b1 + b2).
    """
    A1, b1 = p1
    A2, b2 = p2
    return (A2 @ A1, A2 @ b1 + b2)


def apply_pair(p, h):
    """Apply the affine step p = (a, b) to the state h: a h + b."""
    a, b = p
    return a * h + b


def fold_h0(a, b, h0):
    """Fold a nonzero initial state into the first step.

    ZTF "Scans over vector and matrix states" (the second way of handling
    h_0): replace b_1 by b_1 + a_1 h_0, then scan from zero.  Time is axis 0.
    """
    b = np.array(b, dtype=np.float64, copy=True)
    if h0 is not None:
        b[0] = b[0] + np.asarray(a, dtype=np.float64)[0] * h0
    return b


# ---------------------------------------------------------------------------
# Sequential loop: the recurrence itself (the "recurrent mode").
# ---------------------------------------------------------------------------


def scan_loop(a, b, h0=None):
    """h_t = a_t h_{t-1} + b_t for every channel.

    a, b: [B, T, D]; h0: [B, D] or None (zero, ZTF "The scan for one number of
    state").  Returns (h [B, T, D], h_T [B, D]).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    Bn, T, D = a.shape
    h = np.zeros((Bn, D)) if h0 is None else np.array(h0, dtype=np.float64)
    out = np.empty((Bn, T, D))
    for t in range(T):
        h = a[:, t] * h + b[:, t]
        out[:, t] = h
    return out, h


# ---------------------------------------------------------------------------
# Two parallel scans over the time axis (axis 0), with combine counters.
# ---------------------------------------------------------------------------


class Counter:
    """Counts applications of ``compose`` (one per position per round)."""

    def __init__(self):
        self.combines = 0
        self.rounds = 0


def hillis_steele(a, b, counter: Counter | None = None):
    """Inclusive scan of the pairs (a_t, b_t) along axis 0.

    ZTF "The scan for one number of state" (first parallel scan) and WIKI
    "Blelloch's two sweeps" / its code listing: in round r every position
    combines with the element 2^r places to its left, using the previous
    round's values; positions with no such element keep their value (they
    would combine with the identity).  Returns (A, beta): A_t = a_t...a_1 and
    beta_t = the state at t started from zero.
    """
    A = np.array(a, dtype=np.float64, copy=True)
    Bt = np.array(b, dtype=np.float64, copy=True)
    T = A.shape[0]
    shift = 1
    while shift < T:
        prev = (A[:-shift].copy(), Bt[:-shift].copy())
        cur = (A[shift:].copy(), Bt[shift:].copy())
        # earlier block (prev) on the left
        A[shift:], Bt[shift:] = compose(prev, cur)
        if counter is not None:
            counter.combines += T - shift
            counter.rounds += 1
        shift *= 2
    return A, Bt


def blelloch(a, b, counter: Counter | None = None):
    """Work-efficient inclusive scan along axis 0 (up-sweep, down-sweep).

    ZTF "A vectorized scan for diagonal states" and WIKI "Blelloch's two
    sweeps": pad to a power of two with the identity, sweep up a binary tree
    combining neighbours, set the root to the identity and sweep down handing
    each node the combination of everything to its left (the prefix arriving
    from the left stays the LEFT argument), which gives the exclusive scan;
    one more combine per element turns it into the inclusive scan.
    Counter: up- and down-sweep combines are counted over the padded length,
    the final exclusive-to-inclusive pass over the real length; ``rounds``
    counts the dependent steps of the two sweeps.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    T = a.shape[0]
    n = 1
    while n < T:
        n *= 2
    tail = a.shape[1:]
    A = np.ones((n,) + tail)
    Bt = np.zeros((n,) + tail)
    A[:T] = a
    Bt[:T] = b
    # up-sweep
    d = 1
    while d < n:
        left = np.arange(d - 1, n, 2 * d)
        right = left + d
        A[right], Bt[right] = compose((A[left], Bt[left]), (A[right], Bt[right]))
        if counter is not None:
            counter.combines += len(left)
            counter.rounds += 1
        d *= 2
    # down-sweep: root gets the identity
    A[n - 1], Bt[n - 1] = IDENTITY
    d = n // 2
    while d >= 1:
        left = np.arange(d - 1, n, 2 * d)
        right = left + d
        la, lb = A[left].copy(), Bt[left].copy()
        ra, rb = A[right].copy(), Bt[right].copy()
        # left child receives the parent's prefix; right child receives
        # "prefix, then left subtree": the prefix stays on the left
        A[left], Bt[left] = ra, rb
        A[right], Bt[right] = compose((ra, rb), (la, lb))
        if counter is not None:
            counter.combines += len(left)
            counter.rounds += 1
        d //= 2
    # exclusive -> inclusive: prefix (earlier), then the element itself
    EA, EB = compose((A[:T], Bt[:T]), (a, b))
    if counter is not None:
        counter.combines += T
    return EA, EB


def loop_time0(a, b, counter: Counter | None = None):
    """The loop along axis 0 as a scan of pairs (T - 1 combines)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    A = np.empty_like(a)
    Bt = np.empty_like(b)
    A[0], Bt[0] = a[0], b[0]
    for t in range(1, a.shape[0]):
        A[t], Bt[t] = compose((A[t - 1], Bt[t - 1]), (a[t], b[t]))
        if counter is not None:
            counter.combines += 1
            counter.rounds += 1
    return A, Bt


# ---------------------------------------------------------------------------
# Backward: ZTF "The backward pass is a scan in reverse".  The adjoint
# hbar_t = dL/dh_t obeys the forward recurrence run in reverse time with the
# decays shifted by one place:
#     hbar_T = g_T (+ the gradient dh_T arriving at the returned final state)
#     hbar_t = g_t + a_{t+1} hbar_{t+1}
# and then  db_t = hbar_t,  da_t = hbar_t h_{t-1} (h_0 at t = 1),
#           dh0  = a_1 hbar_1.
# ---------------------------------------------------------------------------


def scan_bwd_loop(a, h, h0, dh, dhT=None):
    """Gradients of a loss L(h, h_T) through the recurrence.

    a, h, dh: [B, T, D] (h is the forward output); h0, dhT: [B, D] or None.
    Returns (da, db, dh0), all float64.
    """
    a = np.asarray(a, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    Bn, T, D = a.shape
    h0 = np.zeros((Bn, D)) if h0 is None else np.asarray(h0, dtype=np.float64)
    hbar = np.zeros((Bn, D)) if dhT is None else np.array(dhT, dtype=np.float64)
    da = np.empty((Bn, T, D))
    db = np.empty((Bn, T, D))
    for t in range(T - 1, -1, -1):
        if t < T - 1:
            hbar = a[:, t + 1] * hbar
        hbar = dh[:, t] + hbar
        db[:, t] = hbar
        da[:, t] = hbar * (h[:, t - 1] if t > 0 else h0)
    dh0 = (a[:, 0] * hbar) if T > 0 else hbar.copy()
    return da, db, dh0


# ---------------------------------------------------------------------------
# Segment products.  ZTF "Long products without underflow": a_{t:s} is the
# product a_t ... a_{s+1} (empty product 1 when t = s).  Built here by
# multiplications only (the first of the page's three safe ways).
# ---------------------------------------------------------------------------


def segment_product_matrix(a1d):
    """T x T lower-triangular M with M[t, s] = a_{t:s} (1-based t, s; the
    diagonal is 1), for a one-dimensional decay sequence (time axis 0)."""
    a1d = np.asarray(a1d, dtype=np.float64)
    T = a1d.shape[0]
    M = np.zeros((T, T))
    for s in range(T):
        p = 1.0
        M[s, s] = 1.0
        for t in range(s + 1, T):
            p = p * a1d[t]
            M[t, s] = p
    return M
