"""Pins for the selective-scan oracle (N state entries per channel, Mamba-1's
recurrence), against things other than itself: the pinned diagonal-scan
oracle on the flattened (channel, entry) states, a path-sum form with no
recurrence, a closed-form geometric series, the no-decay cumulative sum,
stitched pieces, and central finite differences for the backward (CPU)."""

import numpy as np
import pytest

import synthetic as syn
from oracle import scan as oscan
from oracle import sscan as oss

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _one(ci, i=0):
    """Per-sequence float64 views of batch element i."""
    f = lambda v: None if v is None else np.asarray(v, dtype=np.float64)
    return (f(ci.x[i]), f(ci.delta[i]), f(ci.A), f(ci.Bm[i]), f(ci.Cm[i]),
            None if ci.h0 is None else f(ci.h0[i]), f(ci.dy[i]),
            None if ci.dhT is None else f(ci.dhT[i]))


def test_equals_diagonal_scan_on_flattened_states():
    """Every (channel, entry) pair is one scalar recurrence h = a h + b
    (ZTF "Scans over vector and matrix states": a diagonal transition), so the
    pinned diagonal-scan loop over D*N channels, with a = exp(delta A) and
    b = delta B x, gives the same states; y contracts them with C."""
    ci = syn.sscan_inputs(1, 37, 5, 4, 11, A=("uniform", -3.0, -0.05), h0_scale=0.7)
    x, dl, A, Bm, Cm, h0, _, _ = _one(ci)
    T, D = x.shape
    N = A.shape[1]
    a = np.exp(dl[:, :, None] * A[None])            # [T, D, N]
    b = (dl * x)[:, :, None] * Bm[:, None, :]
    h = oscan.scan_loop(a.reshape(1, T, D * N), b.reshape(1, T, D * N),
                        h0.reshape(1, D * N))[0].reshape(T, D, N)
    y_ref = (h * Cm[:, None, :]).sum(axis=2)
    y, hT = oss.sscan_loop(x, dl, A, Bm, Cm, h0)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hT, h[-1], rtol=1e-12, atol=1e-12)


def test_path_sum_form_equals_loop():
    ci = syn.sscan_inputs(1, 13, 3, 5, 12, delta=("loguniform", 1e-2, 1.0),
                          A=("uniform", -2.0, 0.0), h0_scale=1.0)
    x, dl, A, Bm, Cm, h0, _, _ = _one(ci)
    y, hT = oss.sscan_loop(x, dl, A, Bm, Cm, h0)
    y2, hT2 = oss.sscan_matrix_mode(x, dl, A, Bm, Cm, h0)
    np.testing.assert_allclose(y, y2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(hT, hT2, rtol=1e-11, atol=1e-12)


def test_constant_inputs_geometric_series():
    """With delta, x, B, A constant in time, a = exp(delta A) and b = delta B x
    are constant, so h_t = a^t h0 + b (1 - a^t) / (1 - a) (sum of a geometric
    series) and y_t = sum_n C_t[n] h_t[n]."""
    T, D, N = 25, 2, 3
    rng = np.random.default_rng(5)
    dl = np.full((T, D), 0.3)
    x = np.tile(rng.standard_normal(D), (T, 1))
    A = -rng.uniform(0.2, 2.0, size=(D, N))
    Bm = np.tile(rng.standard_normal(N), (T, 1))
    Cm = rng.standard_normal((T, N))
    h0 = rng.standard_normal((D, N))
    a = np.exp(0.3 * A)
    b = 0.3 * x[0][:, None] * Bm[0][None, :]
    t = np.arange(1, T + 1)[:, None, None]
    h = a[None] ** t * h0[None] + b[None] * (1 - a[None] ** t) / (1 - a[None])
    y, hT = oss.sscan_loop(x, dl, A, Bm, Cm, h0)
    np.testing.assert_allclose(y, (h * Cm[:, None, :]).sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hT, h[-1], rtol=1e-12)


def test_no_decay_is_cumulative_sum():
    """A = 0: every decay is 1 and the state is h0 plus the running sum of
    delta B x."""
    ci = syn.sscan_inputs(1, 30, 4, 3, 13, A=("const", 0.0), h0_scale=1.0)
    x, dl, A, Bm, Cm, h0, _, _ = _one(ci)
    b = (dl * x)[:, :, None] * Bm[:, None, :]
    h = h0[None] + np.cumsum(b, axis=0)
    y, hT = oss.sscan_loop(x, dl, A, Bm, Cm, h0)
    np.testing.assert_allclose(y, (h * Cm[:, None, :]).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_stitched_pieces():
    """Running [0, T1) and then [T1, T) from the first piece's final state
    equals one run; in the backward, the second piece's dh0 is the first
    piece's dhT."""
    ci = syn.sscan_inputs(1, 40, 3, 4, 14, A=("uniform", -2.0, -0.1), h0_scale=0.5,
                          dhT_scale=0.5)
    x, dl, A, Bm, Cm, h0, dy, dhT = _one(ci)
    T1 = 17
    y, hT = oss.sscan_loop(x, dl, A, Bm, Cm, h0)
    ya, ha = oss.sscan_loop(x[:T1], dl[:T1], A, Bm[:T1], Cm[:T1], h0)
    yb, hb = oss.sscan_loop(x[T1:], dl[T1:], A, Bm[T1:], Cm[T1:], ha)
    np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hb, hT, rtol=1e-12)
    g = oss.sscan_bwd_loop(x, dl, A, Bm, Cm, h0, dy, dhT)
    gb = oss.sscan_bwd_loop(x[T1:], dl[T1:], A, Bm[T1:], Cm[T1:], ha, dy[T1:], dhT)
    ga = oss.sscan_bwd_loop(x[:T1], dl[:T1], A, Bm[:T1], Cm[:T1], h0, dy[:T1], gb[5])
    for k in (0, 1, 3, 4):
        np.testing.assert_allclose(np.concatenate([ga[k], gb[k]]), g[k], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ga[2] + gb[2], g[2], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ga[5], g[5], rtol=1e-10, atol=1e-12)


def _loss(x, dl, A, Bm, Cm, h0, dy, dhT):
    y, hT = oss.sscan_loop(x, dl, A, Bm, Cm, h0)
    return float((y * dy).sum() + (hT * dhT).sum())


def test_backward_finite_differences():
    """Central differences of L = <y, dy> + <h_T, dh_T> in every input."""
    ci = syn.sscan_inputs(1, 9, 3, 4, 15, delta=("loguniform", 5e-2, 0.8),
                          A=("uniform", -1.5, -0.1), h0_scale=1.0, dhT_scale=1.0)
    x, dl, A, Bm, Cm, h0, dy, dhT = _one(ci)
    grads = oss.sscan_bwd_loop(x, dl, A, Bm, Cm, h0, dy, dhT)
    names = ("x", "delta", "A", "B", "C", "h0")
    args = [x, dl, A, Bm, Cm, h0]
    eps = 1e-6
    for gi, (name, g) in enumerate(zip(names, grads)):
        base = args[gi]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            p = [v.copy() for v in args]
            m = [v.copy() for v in args]
            p[gi][idx] += eps
            m[gi][idx] -= eps
            fd[idx] = (_loss(*p, dy, dhT) - _loss(*m, dy, dhT)) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_backward_state_gradient_equals_diagonal_scan_adjoint():
    """The adjoint of the flattened scalar recurrences, from the pinned
    diagonal-scan backward with upstream gradient C_t[n] dy_t[d] per state,
    gives the same dh0; and the decay-rate gradient dA equals
    sum_t (dL/da_t) a_t delta_t built from that scan's da."""
    ci = syn.sscan_inputs(1, 21, 3, 4, 16, delta=("loguniform", 1e-2, 0.5),
                          A=("uniform", -2.0, -0.1), h0_scale=1.0, dhT_scale=1.0)
    x, dl, A, Bm, Cm, h0, dy, dhT = _one(ci)
    T, D = x.shape
    N = A.shape[1]
    a = np.exp(dl[:, :, None] * A[None])
    b = (dl * x)[:, :, None] * Bm[:, None, :]
    h, _ = oscan.scan_loop(a.reshape(1, T, D * N), b.reshape(1, T, D * N), h0.reshape(1, D * N))
    g = (dy[:, :, None] * Cm[:, None, :]).reshape(1, T, D * N)
    da, db, dh0 = oscan.scan_bwd_loop(a.reshape(1, T, D * N), h, h0.reshape(1, D * N), g,
                                      dhT.reshape(1, D * N))
    dA_ref = (da.reshape(T, D, N) * a * dl[:, :, None]).sum(axis=0)
    r = oss.sscan_bwd_loop(x, dl, A, Bm, Cm, h0, dy, dhT)
    np.testing.assert_allclose(r[5], dh0.reshape(D, N), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r[2], dA_ref, rtol=1e-10, atol=1e-12)


def test_planted_mistake_is_caught(monkeypatch):
    """An oracle whose input term drops the step size (b = B x) must fail the
    geometric-series pin: the pins can tell."""
    def wrong(x, delta, A, Bm):
        x, delta, A, Bm = (np.asarray(v, dtype=np.float64) for v in (x, delta, A, Bm))
        return np.exp(delta[:, :, None] * A[None]), x[:, :, None] * Bm[:, None, :]
    monkeypatch.setattr(oss, "discretize", wrong)
    with pytest.raises(AssertionError):
        test_constant_inputs_geometric_series()


def test_empty_sequence():
    D, N = 3, 2
    h0 = np.ones((D, N))
    y, hT = oss.sscan_loop(np.zeros((0, D)), np.zeros((0, D)), -np.ones((D, N)),
                           np.zeros((0, N)), np.zeros((0, N)), h0)
    assert y.shape == (0, D) and np.array_equal(hT, h0)


def test_c_oracle_matches_numpy():
    from oracle import cref
    ci = syn.sscan_inputs(2, 33, 5, 4, 17, A=("uniform", -2.0, -0.1), h0_scale=0.5,
                          dhT_scale=0.5)
    Bt, T, D = ci.x.shape
    N = ci.A.shape[1]
    chans = np.array([0, 3, 5, 9], dtype=np.int64)
    y, hT = cref.sscan_fwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, chans=chans)
    g = cref.sscan_bwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, ci.dy, ci.dhT, chans=chans)
    yr, hTr = oss.sscan_fwd_batched(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0)
    gr = [oss.sscan_bwd_loop(*_one(ci, b)) for b in range(Bt)]
    for i, c in enumerate(chans):
        b, d = divmod(int(c), D)
        np.testing.assert_allclose(y[i], yr[b, :, d], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(hT[i], hTr[b, d], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g[0][i], gr[b][0][:, d], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g[1][i], gr[b][1][:, d], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g[5][i], gr[b][5][d], rtol=1e-11, atol=1e-12)
    # all channels: dB, dC and the batch-summed dA
    g_all = cref.sscan_bwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, ci.dy, ci.dhT)
    for b in range(Bt):
        np.testing.assert_allclose(g_all[3][b], gr[b][3], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g_all[4][b], gr[b][4], rtol=1e-11, atol=1e-12)
    dA = g_all[2].reshape(Bt, D, N).sum(axis=0)
    np.testing.assert_allclose(dA, sum(r[2] for r in gr), rtol=1e-11, atol=1e-12)
