"""Pins for the diagonal-recurrence oracle (CPU only).

Each test ties ``oracle.scan`` (and the C loops in ``oracle/ref.c``) to
something other than itself: values printed on the pages (tests/golden), two
independent scan algorithms, closed forms, special cases that reduce to numpy
routines, and central finite differences.
"""

import os

import numpy as np
import pytest

from oracle import scan as osc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------------
# pair algebra
# --------------------------------------------------------------------------


def test_worked_composition_and_fold():
    for row in _golden("pair_algebra.txt"):
        if row[0] == "compose":
            a1, b1, a2, b2 = map(float, row[1:5])
            want = tuple(map(float, row[6:8]))
            assert osc.compose((a1, b1), (a2, b2)) == want
            # the reverse order gives a different pair, so the test fixes the order
            assert osc.compose((a2, b2), (a1, b1)) != want
        elif row[0] == "fold":
            h0, a1, b1 = map(float, row[1:4])
            want = float(row[5])
            folded = osc.fold_h0(np.array([a1]), np.array([b1]), h0)
            assert folded[0] == want
            h, _ = osc.scan_loop(np.array([[[a1]]]), np.array([[[b1]]]), np.array([[h0]]))
            assert h[0, 0, 0] == want


def test_identity_two_sided():
    rng = np.random.default_rng(0)
    for _ in range(20):
        p = (rng.uniform(0, 1), rng.normal())
        assert osc.compose(osc.IDENTITY, p) == p
        assert osc.compose(p, osc.IDENTITY) == p


def test_associativity_exact_on_dyadic_values():
    rng = np.random.default_rng(1)
    for _ in range(200):
        ps = [(rng.integers(0, 16) / 16, rng.integers(-64, 64) / 8) for _ in range(3)]
        l = osc.compose(osc.compose(ps[0], ps[1]), ps[2])
        r = osc.compose(ps[0], osc.compose(ps[1], ps[2]))
        assert l == r


def test_associativity_random_float64():
    rng = np.random.default_rng(2)
    ps = [(rng.uniform(0, 1, 100), rng.normal(size=100)) for _ in range(3)]
    l = osc.compose(osc.compose(ps[0], ps[1]), ps[2])
    r = osc.compose(ps[0], osc.compose(ps[1], ps[2]))
    np.testing.assert_allclose(l[0], r[0], rtol=1e-14)
    np.testing.assert_allclose(l[1], r[1], rtol=1e-12, atol=1e-14)


def test_dense_3x3_associative_not_commutative_and_scan():
    rng = np.random.default_rng(3)
    ps = [(rng.normal(size=(3, 3)), rng.normal(size=3)) for _ in range(3)]
    l = osc.compose_dense(osc.compose_dense(ps[0], ps[1]), ps[2])
    r = osc.compose_dense(ps[0], osc.compose_dense(ps[1], ps[2]))
    np.testing.assert_allclose(l[0], r[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l[1], r[1], rtol=1e-12, atol=1e-12)
    ab = osc.compose_dense(ps[0], ps[1])
    ba = osc.compose_dense(ps[1], ps[0])
    assert not np.allclose(ab[0], ba[0])
    # matrix-affine Hillis-Steele (same rounds, dense combine) equals the loop
    T = 13
    As = rng.normal(size=(T, 3, 3)) * 0.5
    bs = rng.normal(size=(T, 3))
    h0 = rng.normal(size=3)
    hs = [(As[t], bs[t]) for t in range(T)]
    shift = 1
    while shift < T:
        hs = hs[:shift] + [osc.compose_dense(hs[t - shift], hs[t]) for t in range(shift, T)]
        shift *= 2
    h = h0
    for t in range(T):
        h = As[t] @ h + bs[t]
        At, bt = hs[t]
        np.testing.assert_allclose(At @ h0 + bt, h, rtol=1e-10, atol=1e-10)


# --------------------------------------------------------------------------
# three scan algorithms agree; combine counts from the pages
# --------------------------------------------------------------------------


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 64, 1000])
def test_loop_hillis_steele_blelloch_agree(T):
    rng = np.random.default_rng(T)
    a = rng.uniform(0.0, 1.0, size=(T, 7))
    b = rng.normal(size=(T, 7))
    h, _ = osc.scan_loop(a[None], b[None])
    h = h[0]
    A1, B1 = osc.hillis_steele(a, b)
    A2, B2 = osc.blelloch(a, b)
    A3, B3 = osc.loop_time0(a, b)
    for Bx in (B1, B2, B3):
        np.testing.assert_allclose(Bx, h, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(A1, np.cumprod(a, axis=0), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(A2, np.cumprod(a, axis=0), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(A3, np.cumprod(a, axis=0), rtol=1e-12, atol=1e-300)


def test_combine_counts_match_pages():
    want = {}
    for alg, T, qty, val in _golden("scan_counts.txt"):
        want[(alg, int(T), qty)] = int(val)
    for T in sorted({k[1] for k in want}):
        a = np.full(T, 0.5)
        b = np.ones(T)
        ch, cb, cl = osc.Counter(), osc.Counter(), osc.Counter()
        osc.hillis_steele(a, b, ch)
        osc.blelloch(a, b, cb)
        osc.loop_time0(a, b, cl)
        n = 1
        while n < T:
            n *= 2
        got = {
            ("blelloch", T, "combines"): cb.combines,
            ("blelloch", T, "up"): n - 1,
            ("blelloch", T, "down"): n - 1,
            ("blelloch", T, "incl"): cb.combines - 2 * (n - 1),
            ("blelloch", T, "depth"): cb.rounds,
            ("hillis_steele", T, "combines"): ch.combines,
            ("hillis_steele", T, "rounds"): ch.rounds,
            ("loop", T, "combines"): cl.combines,
            ("loop", T, "depth"): cl.rounds,
        }
        for key, val in want.items():
            if key[1] == T:
                assert got[key] == val, key


# --------------------------------------------------------------------------
# forward: closed form and special cases
# --------------------------------------------------------------------------


def test_closed_form_prefix_applied_to_h0():
    rng = np.random.default_rng(4)
    T = 40
    a = rng.uniform(0.3, 1.0, T)
    b = rng.normal(size=T)
    h0 = 1.7
    h, hT = osc.scan_loop(a[None, :, None], b[None, :, None], np.array([[h0]]))
    M = osc.segment_product_matrix(a)
    # h_t = a_{t:0} h0 + sum_s a_{t:s} b_s
    pref = np.cumprod(a)
    np.testing.assert_allclose(h[0, :, 0], pref * h0 + M @ b, rtol=1e-12)
    assert hT[0, 0] == h[0, -1, 0]


def test_special_cases_cumsum_and_reset():
    rng = np.random.default_rng(5)
    b = rng.normal(size=(2, 50, 3))
    h0 = rng.normal(size=(2, 3))
    h, _ = osc.scan_loop(np.ones_like(b), b, h0)
    np.testing.assert_allclose(h, np.cumsum(b, axis=1) + h0[:, None, :], rtol=1e-12)
    h, _ = osc.scan_loop(np.zeros_like(b), b, h0)
    np.testing.assert_array_equal(h, b)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------


def _loss(a, b, h0, g, gT):
    h, hT = osc.scan_loop(a, b, h0)
    return np.sum(g * h) + np.sum(gT * hT)


def test_backward_finite_differences_50_steps():
    rng = np.random.default_rng(6)
    T = 50
    a = rng.uniform(0.5, 1.0, (1, T, 2))
    b = rng.normal(size=(1, T, 2))
    h0 = rng.normal(size=(1, 2))
    g = rng.normal(size=(1, T, 2))
    gT = rng.normal(size=(1, 2))
    h, _ = osc.scan_loop(a, b, h0)
    da, db, dh0 = osc.scan_bwd_loop(a, h, h0, g, gT)
    eps = 1e-6

    def fd(x, idx, which):
        xp = x.copy()
        xm = x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        args_p = dict(a=a, b=b, h0=h0)
        args_m = dict(a=a, b=b, h0=h0)
        args_p[which] = xp
        args_m[which] = xm
        return (_loss(args_p["a"], args_p["b"], args_p["h0"], g, gT)
                - _loss(args_m["a"], args_m["b"], args_m["h0"], g, gT)) / (2 * eps)

    for t in (0, 1, 17, T - 2, T - 1):
        for d in range(2):
            assert fd(a, (0, t, d), "a") == pytest.approx(da[0, t, d], rel=1e-6, abs=1e-8)
            assert fd(b, (0, t, d), "b") == pytest.approx(db[0, t, d], rel=1e-6, abs=1e-8)
    for d in range(2):
        assert fd(h0, (0, d), "h0") == pytest.approx(dh0[0, d], rel=1e-6, abs=1e-8)


def test_backward_exact_linear_maps():
    # h is linear in (b, h0): h = M b + a_{t:0} h0, so db = M^T g (+ the final
    # state's row) and dh0 = sum_t a_{t:0} g_t + a_{T:0} dh_T.
    rng = np.random.default_rng(7)
    T = 30
    a = rng.uniform(0.2, 1.0, T)
    b = rng.normal(size=T)
    g = rng.normal(size=T)
    gT = 0.7
    h0 = -0.4
    h, _ = osc.scan_loop(a[None, :, None], b[None, :, None], np.array([[h0]]))
    da, db, dh0 = osc.scan_bwd_loop(a[None, :, None], h, np.array([[h0]]),
                                     g[None, :, None], np.array([[gT]]))
    M = osc.segment_product_matrix(a)
    np.testing.assert_allclose(db[0, :, 0], M.T @ g + gT * M[T - 1], rtol=1e-12)
    pref = np.cumprod(a)
    assert dh0[0, 0] == pytest.approx(pref @ g + pref[-1] * gT, rel=1e-12)


def test_backward_no_decay_is_reverse_cumsum():
    rng = np.random.default_rng(8)
    g = rng.normal(size=(1, 25, 4))
    a = np.ones_like(g)
    h, _ = osc.scan_loop(a, rng.normal(size=g.shape))
    _, db, _ = osc.scan_bwd_loop(a, h, None, g)
    np.testing.assert_allclose(db, np.cumsum(g[:, ::-1], axis=1)[:, ::-1], rtol=1e-12)


def test_backward_empty_sequence():
    a = np.zeros((2, 0, 3))
    dhT = np.arange(6.0).reshape(2, 3)
    da, db, dh0 = osc.scan_bwd_loop(a, a, None, a, dhT)
    assert da.shape == (2, 0, 3) and db.shape == (2, 0, 3)
    np.testing.assert_array_equal(dh0, dhT)


def test_planted_mistakes_are_caught():
    """A plausible mistake anywhere in the backward fails a pin: an unshifted
    decay (a_t instead of a_{t+1}) breaks the exact linear map."""
    rng = np.random.default_rng(9)
    T = 12
    a = rng.uniform(0.2, 0.9, T)
    g = rng.normal(size=T)
    M = osc.segment_product_matrix(a)
    hbar = 0.0
    wrong = np.empty(T)
    for t in range(T - 1, -1, -1):
        hbar = g[t] + a[t] * hbar if t < T - 1 else g[t]
        wrong[t] = hbar
    assert not np.allclose(wrong, M.T @ g)
    # composing in the wrong order fails the worked example
    a1, b1, a2, b2 = 0.5, 1.0, 0.5, 0.0
    assert (a1 * a2, a1 * b2 + b1) != (0.25, 0.5)


# --------------------------------------------------------------------------
# the C loops equal the (pinned) numpy definitions
# --------------------------------------------------------------------------


def test_c_oracle_matches_numpy(coracle):
    rng = np.random.default_rng(10)
    B, T, D = 3, 97, 5
    a = rng.uniform(0, 1, (B, T, D)).astype(np.float32)
    b = rng.normal(size=(B, T, D)).astype(np.float32)
    h0 = rng.normal(size=(B, D)).astype(np.float32)
    dh = rng.normal(size=(B, T, D)).astype(np.float32)
    dhT = rng.normal(size=(B, D)).astype(np.float32)
    h_ref, hT_ref = osc.scan_loop(a, b, h0)
    h, hT = coracle.scan_fwd(a, b, h0)
    np.testing.assert_allclose(h, h_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hT, hT_ref, rtol=1e-13, atol=1e-13)
    h32 = h.astype(np.float32)
    da_ref, db_ref, dh0_ref = osc.scan_bwd_loop(a, h32, h0, dh, dhT)
    da, db, dh0 = coracle.scan_bwd(a, h32, h0, dh, dhT)
    np.testing.assert_allclose(da, da_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(db, db_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dh0, dh0_ref, rtol=1e-13, atol=1e-13)
    # a channel block
    h2, hT2 = coracle.scan_fwd(a, b, h0, brange=(1, 3), drange=(2, 4))
    np.testing.assert_allclose(h2, h_ref[1:3, :, 2:4], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(hT2, hT_ref[1:3, 2:4], rtol=1e-13, atol=1e-13)
