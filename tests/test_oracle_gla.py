"""Pins of the float64 oracle for one decay per key dimension (CPU).

Each pin ties oracle/gla.py to something other than itself:
  * a decay that is the same in every key dimension reduces the vector form to
    the scalar recurrence of oracle/attn.py (pinned on its own);
  * the recurrence splits exactly into dk independent width-1 problems of the
    scalar form (row d of the state only ever sees dimension d of q, k, l);
  * the brute-force matrix mode and the chunkwise form equal the loop;
  * every gradient of the adjoint loop matches central finite differences;
  * the closed-form vector decay gradient equals the direct one;
  * the C loops (oracle/ref.c) equal the numpy ones.
"""

import numpy as np
import pytest

from oracle import attn, gla


def _rand(T, dk, dv, seed, scale=0.5, l_lo=-1.0, l_hi=0.0):
    g = np.random.default_rng(seed)
    q = g.standard_normal((T, dk)) * scale
    k = g.standard_normal((T, dk)) * scale
    v = g.standard_normal((T, dv))
    l = g.uniform(l_lo, l_hi, (T, dk))
    S0 = g.standard_normal((dk, dv)) * 0.3
    return q, k, v, l, S0


def test_equal_decays_reduce_to_scalar():
    q, k, v, l, S0 = _rand(37, 5, 4, 1)
    ls = l[:, 0]
    lv = np.repeat(ls[:, None], 5, axis=1)
    o_v, S_v = gla.gla_loop(q, k, v, lv, S0)
    o_s, S_s = attn.la_loop(q, k, v, ls, S0)
    np.testing.assert_allclose(o_v, o_s, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_v, S_s, rtol=1e-12, atol=1e-12)
    dO = np.random.default_rng(2).standard_normal((37, 4))
    dST = np.random.default_rng(3).standard_normal((5, 4))
    gv = gla.gla_bwd_loop(q, k, v, lv, S0, dO, dST)
    gs = attn.la_bwd_loop(q, k, v, ls, S0, dO, dST)
    for a, b in zip(gv[:3] + gv[4:], gs[:3] + gs[4:]):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)
    # the scalar log decay feeds every dimension: its gradient is the sum
    np.testing.assert_allclose(gv[3].sum(axis=1), gs[3], rtol=1e-11, atol=1e-11)


def test_sum_of_width_one_problems():
    """Row d of the state evolves as S[d] <- a[d] S[d] + k[d] v, so the output
    is a sum over d of scalar problems with one key dimension."""
    T, dk, dv = 29, 4, 3
    q, k, v, l, S0 = _rand(T, dk, dv, 4, l_lo=-3.0)
    dO = np.random.default_rng(5).standard_normal((T, dv))
    dST = np.random.default_rng(6).standard_normal((dk, dv))
    o, ST = gla.gla_loop(q, k, v, l, S0)
    dq, dkk, dvv, dl, dS0 = gla.gla_bwd_loop(q, k, v, l, S0, dO, dST)
    o_sum = np.zeros((T, dv))
    dv_sum = np.zeros((T, dv))
    for d in range(dk):
        sl = slice(d, d + 1)
        o_d, S_d = attn.la_loop(q[:, sl], k[:, sl], v, l[:, d], S0[sl])
        o_sum += o_d
        np.testing.assert_allclose(ST[sl], S_d, rtol=1e-12, atol=1e-12)
        g = attn.la_bwd_loop(q[:, sl], k[:, sl], v, l[:, d], S0[sl], dO, dST[sl])
        np.testing.assert_allclose(dq[:, sl], g[0], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(dkk[:, sl], g[1], rtol=1e-11, atol=1e-11)
        dv_sum += g[2]
        np.testing.assert_allclose(dl[:, d], g[3], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(dS0[sl], g[4], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(o, o_sum, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dvv, dv_sum, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("T,Tc", [(1, 64), (9, 4), (64, 64), (150, 64), (70, 16), (33, 1)])
def test_chunkwise_equals_loop(T, Tc):
    q, k, v, l, S0 = _rand(T, 6, 5, 10 + T, l_lo=-2.0)
    o_r, S_r = gla.gla_loop(q, k, v, l, S0)
    o_c, S_c = gla.gla_chunkwise(q, k, v, l, S0, Tc=Tc)
    np.testing.assert_allclose(o_c, o_r, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(S_c, S_r, rtol=1e-10, atol=1e-10)


def test_matrix_mode_equals_loop():
    q, k, v, l, S0 = _rand(23, 4, 3, 20)
    for s0 in (None, S0):
        o_r, S_r = gla.gla_loop(q, k, v, l, s0)
        o_m, S_m = gla.gla_matrix_mode(q, k, v, l, s0)
        np.testing.assert_allclose(o_m, o_r, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(S_m, S_r, rtol=1e-11, atol=1e-11)


def test_backward_finite_differences():
    T, dk, dv = 6, 3, 2
    q, k, v, l, S0 = _rand(T, dk, dv, 30, l_lo=-1.5)
    g = np.random.default_rng(31)
    W = g.standard_normal((T, dv))
    W2 = g.standard_normal((dk, dv))

    def loss(q_, k_, v_, l_, S0_):
        o, ST = gla.gla_loop(q_, k_, v_, l_, S0_)
        return np.sum(o * W) + np.sum(ST * W2)

    grads = gla.gla_bwd_loop(q, k, v, l, S0, W, W2)
    args = [q, k, v, l, S0]
    order = [0, 1, 2, 3, 4]
    h = 1e-6
    for gi, ai in zip(grads, order):
        x = args[ai]
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = list(args)
            am = list(args)
            ap[ai] = xp
            am[ai] = xm
            num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        np.testing.assert_allclose(gi, num, rtol=1e-6, atol=1e-7)


def test_closed_form_dlog_equals_direct():
    T, dk, dv = 40, 5, 4
    q, k, v, l, S0 = _rand(T, dk, dv, 40, l_lo=-2.5)
    g = np.random.default_rng(41)
    dO = g.standard_normal((T, dv))
    for dST in (None, g.standard_normal((dk, dv))):
        dq, dkk, _, dl, _ = gla.gla_bwd_loop(q, k, v, l, S0, dO, dST)
        _, ST = gla.gla_loop(q, k, v, l, S0)
        dl_c = gla.gla_dlog_closed_form(q, k, dq, dkk, ST, dST)
        np.testing.assert_allclose(dl_c, dl, rtol=1e-9, atol=1e-10)


def test_stitched_pieces():
    """Two pieces run back to back with the state passed between them give the
    one-piece result; the backward chains dS0 of the second piece into dS_T of
    the first."""
    T, dk, dv, s = 50, 4, 3, 21
    q, k, v, l, S0 = _rand(T, dk, dv, 50)
    dO = np.random.default_rng(51).standard_normal((T, dv))
    o, ST = gla.gla_loop(q, k, v, l, S0)
    o1, S1 = gla.gla_loop(q[:s], k[:s], v[:s], l[:s], S0)
    o2, S2 = gla.gla_loop(q[s:], k[s:], v[s:], l[s:], S1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, ST, rtol=1e-12, atol=1e-12)
    full = gla.gla_bwd_loop(q, k, v, l, S0, dO)
    g2 = gla.gla_bwd_loop(q[s:], k[s:], v[s:], l[s:], S1, dO[s:])
    g1 = gla.gla_bwd_loop(q[:s], k[:s], v[:s], l[:s], S0, dO[:s], g2[4])
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2), ("dl", 3)):
        np.testing.assert_allclose(np.concatenate([g1[i], g2[i]]), full[i],
                                   rtol=1e-11, atol=1e-11, err_msg=name)
    np.testing.assert_allclose(g1[4], full[4], rtol=1e-11, atol=1e-11)


def test_c_oracle_matches_numpy():
    from oracle import cref
    import synthetic as syn
    B, H, T, DK, DV = 1, 2, 70, 8, 4
    ci = syn.gla_inputs(B, H, T, DK, DV, 60, S0_scale=0.2, dST_scale=0.3)
    f = lambda bits: syn.bf16_bits_to_f64(bits)
    o_c, ST_c = cref.gla_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0)
    g_c = cref.gla_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST)
    for hd in range(B * H):
        b, h = divmod(hd, H)
        args = (f(ci.q[b, h]), f(ci.k[b, h]), f(ci.v[b, h]), ci.l[b, h].astype(np.float64),
                ci.S0[b, h].astype(np.float64))
        o_r, ST_r = gla.gla_loop(*args)
        np.testing.assert_allclose(o_c[hd], o_r, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(ST_c[hd], ST_r, rtol=1e-12, atol=1e-12)
        g_r = gla.gla_bwd_loop(*args, f(ci.dO[b, h]), ci.dST[b, h].astype(np.float64))
        for a, r in zip(g_c, g_r):
            np.testing.assert_allclose(a[hd], r, rtol=1e-11, atol=1e-11)
