"""The float32 facts the kernels' decay handling rests on (CPU only).

ZTF = "Parallel scan" (zerotofrontier.app, ssm/parallel-scan), section "Long
products without underflow".  The values are in tests/golden/float32_facts.txt.
These tests reproduce the page's numbers with IEEE float32 arithmetic in
numpy, and show the two unsafe segment-product formulas failing where the
in-window log sums the chunk kernels use stay accurate.
"""

import os

import numpy as np

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    out = {}
    with open(os.path.join(GOLD, "float32_facts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = float(v)
    return out


def _running_product(x, n):
    p = np.float32(1.0)
    out = np.empty(n + 1, dtype=np.float32)
    out[0] = p
    with np.errstate(under="ignore"):
        for t in range(1, n + 1):
            p = np.float32(p * np.float32(x))
            out[t] = p
    return out


def test_product_of_09_goes_subnormal_and_sticks():
    f = _facts()
    P = _running_product(0.9, 1200)
    tiny = np.finfo(np.float32).tiny
    first_sub = int(np.argmax(P < tiny))
    assert first_sub == int(f["p09_first_subnormal_step"])
    stuck = next(t for t in range(1, 1199) if P[t + 1] == P[t])
    assert stuck == int(f["p09_first_stuck_step"])
    assert abs(float(P[stuck]) - f["p09_stuck_value"]) < 0.1e-45
    assert P[1100] / P[1000] == f["p09_ratio_1100_1000"]


def test_product_of_e_minus_half_sticks_after_206_steps():
    f = _facts()
    P = _running_product(np.exp(np.float32(-0.5)), 400)
    n = int(f["pe05_stuck_after"])
    assert P[n + 1] == P[n]
    assert all(P[t + 1] != P[t] for t in range(n))


def test_long_cumsum_loses_precision_window_sum_does_not():
    rng = np.random.default_rng(0)
    T = 100_000
    l = -rng.uniform(0.0, 0.212, T)       # mean log decay about -0.106
    S = np.cumsum(l.astype(np.float32), dtype=np.float32)
    assert -11_000 < S[-1] < -10_000
    s, t = T - 21, T - 1                   # a 20-step segment at the end
    exact = np.sum(l[s + 1:t + 1])
    long_diff = np.float64(S[t]) - np.float64(S[s])
    window = np.float64(np.sum(l[s + 1:t + 1].astype(np.float32), dtype=np.float32))
    assert abs(np.expm1(long_diff - exact)) > 1e-4      # several 1e-4 .. 1e-3
    assert abs(np.expm1(window - exact)) < 1e-6


def test_window_sums_stay_in_fine_float32_spacing():
    f = _facts()
    # 64 decays above 0.5: the in-chunk cumulative log stays above 64 log 0.5
    floor = 64 * np.log(0.5)
    assert floor > f["window_sum_floor"]
    spacing = float(np.spacing(np.float32(f["window_sum_floor"])))
    assert spacing < 1.1 * f["window_spacing"]
