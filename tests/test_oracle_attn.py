"""Pins for the matrix-state (linear attention) oracle (CPU only).

``oracle.attn`` is tied to things other than itself: the brute-force T x T
matrix mode, special cases with closed forms (no decay, constant decay as
powers), the chunkwise algorithm at its two limits and in between, central
finite differences of a scalar loss, and the exact linear maps of the
backward.  The C loops in ``oracle/ref.c`` are then checked against the
pinned numpy definitions.
"""

import numpy as np
import pytest

from oracle import attn as oa


def _rand(T, dk, dv, seed, lo=-0.3, hi=0.0, S0=True):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(T, dk))
    k = rng.normal(size=(T, dk))
    v = rng.normal(size=(T, dv))
    l = rng.uniform(lo, hi, T)
    S = rng.normal(size=(dk, dv)) if S0 else None
    return q, k, v, l, S


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------


@pytest.mark.parametrize("T,S0", [(1, False), (7, True), (33, False), (64, True)])
def test_loop_equals_matrix_mode(T, S0):
    q, k, v, l, S = _rand(T, 5, 3, T, S0=S0)
    o1, S1 = oa.la_loop(q, k, v, l, S)
    o2, S2 = oa.la_matrix_mode(q, k, v, l, S)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(S1, S2, rtol=1e-11, atol=1e-11)


def test_no_decay_is_causal_linear_attention():
    q, k, v, _, _ = _rand(20, 4, 6, 1)
    o, ST = oa.la_loop(q, k, v, np.zeros(20))
    np.testing.assert_allclose(o, ((q @ k.T) * np.tril(np.ones((20, 20)))) @ v, rtol=1e-12)
    np.testing.assert_allclose(ST, k.T @ v, rtol=1e-12)


def test_constant_decay_powers():
    # LA2 Eq. 4 / Eq. 7: o_t = q_t sum_{s<=t} lambda^{t-s} k_s^T v_s
    q, k, v, _, _ = _rand(25, 3, 4, 2)
    lam = 0.9
    o, _ = oa.la_loop(q, k, v, np.full(25, np.log(lam)))
    want = np.array([q[t] @ sum(lam ** (t - s) * np.outer(k[s], v[s]) for s in range(t + 1))
                     for t in range(25)])
    np.testing.assert_allclose(o, want, rtol=1e-11)


@pytest.mark.parametrize("T,Tc", [(37, 1), (37, 4), (37, 16), (37, 37), (64, 64), (130, 64), (5, 64)])
def test_chunkwise_equals_recurrence(T, Tc):
    q, k, v, l, S = _rand(T, 6, 4, T + Tc)
    o1, S1 = oa.la_loop(q, k, v, l, S)
    o2, S2 = oa.la_chunkwise(q, k, v, l, S, Tc=Tc)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(S2, S1, rtol=1e-10, atol=1e-10)


def test_chunkwise_limits():
    q, k, v, l, _ = _rand(12, 3, 3, 5)
    # T_c = T with S0 = 0: the inter-chunk term vanishes; the quadratic mode
    o_full, _ = oa.la_chunkwise(q, k, v, l, None, Tc=12)
    M = oa.decay_matrix(l)
    np.testing.assert_allclose(o_full, ((q @ k.T) * M) @ v, rtol=1e-12)
    # T_c = 1: every chunk is one token; the recurrence
    o1, S1 = oa.la_chunkwise(q, k, v, l, None, Tc=1)
    o2, S2 = oa.la_loop(q, k, v, l, None)
    np.testing.assert_allclose(o1, o2, rtol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=1e-12)


def test_la2_printed_lambda_reading():
    """LA2 prints Lambda = diag(lambda^0..lambda^{B-1}).  With S0 = 0 it gives the
    same outputs but carries the state decayed once too often (S_T off by a
    factor lambda); a nonzero S0 is then misapplied.  The reading that
    follows ZTF's three decays (lambda_1 includes the first token) matches the
    recurrence in all three respects."""
    T, Tc, lam = 40, 8, 0.8
    q, k, v, _, S = _rand(T, 3, 2, 11)
    l = np.full(T, np.log(lam))
    o_ref, S_ref = oa.la_loop(q, k, v, l, None)
    o_p, S_p = oa.la_chunkwise(q, k, v, l, None, Tc=Tc, la2_printed_lambda=True)
    np.testing.assert_allclose(o_p, o_ref, rtol=1e-11)
    np.testing.assert_allclose(S_p, lam * S_ref, rtol=1e-11)
    assert not np.allclose(S_p, S_ref)
    o_ref2, _ = oa.la_loop(q, k, v, l, S)
    o_p2, _ = oa.la_chunkwise(q, k, v, l, S, Tc=Tc, la2_printed_lambda=True)
    assert not np.allclose(o_p2, o_ref2)
    o_ok, S_ok = oa.la_chunkwise(q, k, v, l, S, Tc=Tc)
    np.testing.assert_allclose(o_ok, o_ref2, rtol=1e-11)


def test_stitched_pieces_equal_whole():
    # ZTF "Scans over vector and matrix states": a piece starts from the state
    # where the previous one ended.
    q, k, v, l, S = _rand(50, 4, 3, 12)
    o, ST = oa.la_loop(q, k, v, l, S)
    o1, S1 = oa.la_loop(q[:23], k[:23], v[:23], l[:23], S)
    o2, S2 = oa.la_loop(q[23:], k[23:], v[23:], l[23:], S1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-12)
    np.testing.assert_allclose(S2, ST, rtol=1e-12)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------


def _loss(q, k, v, l, S0, dO, dST):
    o, ST = oa.la_loop(q, k, v, l, S0)
    return np.sum(o * dO) + np.sum(ST * dST)


def test_backward_finite_differences():
    T, dk, dv = 9, 3, 2
    q, k, v, l, S0 = _rand(T, dk, dv, 21, lo=-0.7, hi=-0.05)
    rng = np.random.default_rng(22)
    dO = rng.normal(size=(T, dv))
    dST = rng.normal(size=(dk, dv))
    dq, dk_, dv_, dl, dS0 = oa.la_bwd_loop(q, k, v, l, S0, dO, dST)
    base = dict(q=q, k=k, v=v, l=l, S0=S0)
    grads = dict(q=dq, k=dk_, v=dv_, l=dl, S0=dS0)
    eps = 1e-6
    for name, x in base.items():
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap = dict(base, **{name: xp})
            am = dict(base, **{name: xm})
            num = (_loss(ap["q"], ap["k"], ap["v"], ap["l"], ap["S0"], dO, dST)
                   - _loss(am["q"], am["k"], am["v"], am["l"], am["S0"], dO, dST)) / (2 * eps)
            assert num == pytest.approx(grads[name][idx], rel=1e-6, abs=1e-7), (name, idx)


def test_closed_form_decay_gradient_equals_direct():
    q, k, v, l, S0 = _rand(70, 5, 4, 31, lo=-0.4, hi=0.0)
    rng = np.random.default_rng(32)
    dO = rng.normal(size=(70, 4))
    dST = rng.normal(size=(5, 4))
    dq, dk, _, dl, _ = oa.la_bwd_loop(q, k, v, l, S0, dO, dST)
    _, ST = oa.la_loop(q, k, v, l, S0)
    np.testing.assert_allclose(oa.dlog_closed_form(q, k, dq, dk, ST, dST), dl,
                               rtol=1e-9, atol=1e-9)
    # without the final-state term the closed form is wrong when dS_T != 0
    assert not np.allclose(oa.dlog_closed_form(q, k, dq, dk), dl)


def test_backward_exact_linear_maps():
    # o and S_T are linear in V and S0:
    #   dV  = (Q K^T (.) M)^T dO + diag(a_{T:s}) K dS_T
    #   dS0 = sum_t a_{t:0} q_t dO_t^T + a_{T:0} dS_T
    T = 30
    q, k, v, l, S0 = _rand(T, 4, 3, 41)
    rng = np.random.default_rng(42)
    dO = rng.normal(size=(T, 3))
    dST = rng.normal(size=(4, 3))
    _, _, dv, _, dS0 = oa.la_bwd_loop(q, k, v, l, S0, dO, dST)
    M = oa.decay_matrix(l)
    want_dv = ((q @ k.T) * M).T @ dO + (k * M[T - 1][:, None]) @ dST
    np.testing.assert_allclose(dv, want_dv, rtol=1e-11, atol=1e-11)
    P = oa.prefix_decay(l)
    want_dS0 = (q * P[:, None]).T @ dO + P[-1] * dST
    np.testing.assert_allclose(dS0, want_dS0, rtol=1e-11, atol=1e-11)


def test_backward_constant_decay_la2_per_token():
    # LA2 Eq. 11-12: dq_t = do_t kv_t^T; dkv_t = sum_{s>=t} lambda^{s-t} q_s^T do_s;
    # dk_t = v_t dkv_t^T; dv_t = k_t dkv_t
    T, lam = 16, 0.85
    q, k, v, _, _ = _rand(T, 3, 2, 51)
    dO = np.random.default_rng(52).normal(size=(T, 2))
    l = np.full(T, np.log(lam))
    dq, dk, dv, _, _ = oa.la_bwd_loop(q, k, v, l, None, dO)
    states = oa.la_loop_states(q, k, v, l)
    for t in range(T):
        dkv = sum(lam ** (s - t) * np.outer(q[s], dO[s]) for s in range(t, T))
        np.testing.assert_allclose(dq[t], states[t + 1] @ dO[t], rtol=1e-11)
        np.testing.assert_allclose(dk[t], dkv @ v[t], rtol=1e-11)
        np.testing.assert_allclose(dv[t], dkv.T @ k[t], rtol=1e-11)


def test_planted_mistake_in_backward_is_caught():
    """Reading the next state's decay at the wrong step (a_t instead of
    a_{t+1}) changes the value gradient, so the exact linear map rejects it."""
    T = 12
    q, k, v, l, _ = _rand(T, 3, 2, 61)
    dO = np.random.default_rng(62).normal(size=(T, 2))
    a = np.exp(l)
    Sbar = np.zeros((3, 2))
    wrong = np.empty((T, 2))
    for t in range(T - 1, -1, -1):
        Sbar = (a[t] * Sbar if t < T - 1 else Sbar) + np.outer(q[t], dO[t])
        wrong[t] = Sbar.T @ k[t]
    M = oa.decay_matrix(l)
    assert not np.allclose(wrong, ((q @ k.T) * M).T @ dO)


# --------------------------------------------------------------------------
# the C loops equal the pinned numpy definitions (bf16 inputs, fp32 decays)
# --------------------------------------------------------------------------


def _bf16(x):
    from synthetic import bf16_bits_from_f32
    return bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("T,dk,dv", [(1, 4, 3), (150, 8, 5), (64, 16, 16)])
def test_c_oracle_matches_numpy(coracle, T, dk, dv):
    from synthetic import bf16_bits_to_f64
    rng = np.random.default_rng(T)
    B, H = 2, 2
    q = _bf16(rng.normal(size=(B, H, T, dk)) * 0.3)
    k = _bf16(rng.normal(size=(B, H, T, dk)) * 0.3)
    v = _bf16(rng.normal(size=(B, H, T, dv)))
    l = rng.uniform(-0.5, 0, (B, H, T)).astype(np.float32)
    S0 = rng.normal(size=(B, H, dk, dv)).astype(np.float32)
    dO = _bf16(rng.normal(size=(B, H, T, dv)))
    dST = rng.normal(size=(B, H, dk, dv)).astype(np.float32)
    Q, K, V, DO = (bf16_bits_to_f64(x) for x in (q, k, v, dO))
    o_ref, ST_ref = oa.la_fwd_batched(Q, K, V, l, S0)
    o, ST = coracle.la_fwd(q, k, v, l, S0)
    np.testing.assert_allclose(o.reshape(o_ref.shape), o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ST.reshape(ST_ref.shape), ST_ref, rtol=1e-12, atol=1e-12)
    ref = oa.la_bwd_batched(Q, K, V, l, S0, DO, dST)
    got = coracle.la_bwd(q, k, v, l, S0, dO, dST)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g.reshape(r.shape), r, rtol=1e-11, atol=1e-11)
    # a subset of heads, no S0 / dST
    o_ref, _ = oa.la_fwd_batched(Q, K, V, l, None)
    o, _ = coracle.la_fwd(q, k, v, l, None, heads=[3, 1])
    np.testing.assert_allclose(o[0], o_ref[1, 1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o[1], o_ref[0, 1], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# exact resets: l_t = -inf (a_t = 0) clears the state before step t's write
# --------------------------------------------------------------------------


def _with_resets(T, seed, at):
    q, k, v, l, S = _rand(T, 5, 4, seed)
    l = l.copy()
    l[list(at)] = -np.inf
    return q, k, v, l, S


@pytest.mark.parametrize("at", [(0,), (9,), (9, 10), (17, 40, 63), (5, 64, 65, 90)])
def test_reset_splits_the_sequence(at):
    """A reset at u makes steps u.. a fresh sequence from a zero state (the
    write at u itself survives): the whole run equals the run on steps u..
    alone, for the recurrence, the T x T matrix mode and the chunkwise form."""
    T = 100
    q, k, v, l, S = _with_resets(T, 40 + len(at), at)
    u = max(at)
    o_tail, S_tail = oa.la_loop(q[u:], k[u:], v[u:], l[u:], None)
    for fn in (oa.la_loop, oa.la_matrix_mode,
               lambda *x: oa.la_chunkwise(*x, Tc=16), lambda *x: oa.la_chunkwise(*x, Tc=64)):
        o, ST = fn(q, k, v, l, S)
        assert np.isfinite(o).all() and np.isfinite(ST).all()
        np.testing.assert_allclose(o[u:], o_tail, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(ST, S_tail, rtol=1e-11, atol=1e-11)
    # before the first reset nothing changes
    u0 = min(at)
    if u0 > 0:
        o_head, _ = oa.la_loop(q[:u0], k[:u0], v[:u0], l[:u0], S)
        o, _ = oa.la_loop(q, k, v, l, S)
        np.testing.assert_allclose(o[:u0], o_head, rtol=1e-12, atol=1e-12)


def test_reset_backward():
    """With resets: the adjoint loop gives zero gradient to the log decay of a
    reset step (a_u = 0 scales every path through it); nothing after the
    first reset reaches the steps before it or the initial state; and the
    closed-form decay gradient still equals the direct one."""
    T = 90
    at = (30, 31, 70)
    q, k, v, l, S0 = _with_resets(T, 7, at)
    rng = np.random.default_rng(8)
    dO = rng.normal(size=(T, 4))
    dST = rng.normal(size=(5, 4))
    dq, dk, dv, dl, dS0 = oa.la_bwd_loop(q, k, v, l, S0, dO, dST)
    for x in (dq, dk, dv, dl, dS0):
        assert np.isfinite(x).all()
    assert all(dl[u] == 0.0 for u in at)
    # the first piece alone, with no gradient arriving after it
    dq1, dk1, dv1, _, dS01 = oa.la_bwd_loop(q[:30], k[:30], v[:30], l[:30], S0, dO[:30], None)
    np.testing.assert_allclose(dS0, dS01, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dq[:30], dq1, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dk[:30], dk1, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dv[:30], dv1, rtol=1e-11, atol=1e-11)
    _, ST = oa.la_loop(q, k, v, l, S0)
    np.testing.assert_allclose(oa.dlog_closed_form(q, k, dq, dk, ST, dST), dl,
                               rtol=1e-9, atol=1e-9)


def test_c_oracle_resets(coracle):
    from synthetic import bf16_bits_to_f64
    rng = np.random.default_rng(5)
    B, H, T, dk, dv = 1, 2, 130, 8, 8
    q = _bf16(rng.normal(size=(B, H, T, dk)) * 0.3)
    k = _bf16(rng.normal(size=(B, H, T, dk)) * 0.3)
    v = _bf16(rng.normal(size=(B, H, T, dv)))
    l = rng.uniform(-0.5, 0, (B, H, T)).astype(np.float32)
    l[0, 0, [0, 64, 65]] = -np.inf
    l[0, 1, [63, 100]] = -np.inf
    S0 = rng.normal(size=(B, H, dk, dv)).astype(np.float32)
    dO = _bf16(rng.normal(size=(B, H, T, dv)))
    dST = rng.normal(size=(B, H, dk, dv)).astype(np.float32)
    Q, K, V, DO = (bf16_bits_to_f64(x) for x in (q, k, v, dO))
    o_ref, ST_ref = oa.la_fwd_batched(Q, K, V, l, S0)
    o, ST = coracle.la_fwd(q, k, v, l, S0)
    np.testing.assert_allclose(o.reshape(o_ref.shape), o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ST.reshape(ST_ref.shape), ST_ref, rtol=1e-12, atol=1e-12)
    ref = oa.la_bwd_batched(Q, K, V, l, S0, DO, dST)
    got = coracle.la_bwd(q, k, v, l, S0, dO, dST)
    for g, r in zip(got, ref):
        assert np.isfinite(g).all()
        np.testing.assert_allclose(g.reshape(r.shape), r, rtol=1e-11, atol=1e-11)
