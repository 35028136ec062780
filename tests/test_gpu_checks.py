"""Device-side checks of the log decays (cla_check_log_decay) and what the
scalar chunkwise call does with a decay it does not accept (GPU).

The counts are integers and are compared exactly with numpy's count of the
same values; the opt-in check of the Python calls raises before any kernel
of the call runs.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _counts_np(x):
    x = np.asarray(x, dtype=np.float32)
    return {"nan": int(np.isnan(x).sum()), "posinf": int(np.isposinf(x).sum()),
            "positive": int(((x > 0) & np.isfinite(x)).sum()), "neginf": int(np.isneginf(x).sum())}


@pytest.mark.parametrize("n", [0, 1, 255, 256, 257, 4096 * 257 + 3, 3_000_017])
def test_counts_match_numpy(n):
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, say
    rng = np.random.default_rng(7000 + n % 97)
    x = (rng.standard_normal(n) * 3).astype(np.float32)
    # sprinkle every kind of value, including at the two ends
    special = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-38, -1e-38, 5.0], np.float32)
    if n:
        idx = rng.integers(0, n, size=min(n, 64))
        x[idx] = special[rng.integers(0, len(special), size=len(idx))]
        x[0] = np.nan
        x[-1] = np.inf
    say(f"[checks] n={n}")
    got = cla.log_decay_counts(torch.from_numpy(x).to(dev()))
    assert got == _counts_np(x)


def test_check_rules_and_opt_in():
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev
    d = dev()
    ok_scalar = torch.tensor([-0.5, 0.0, -np.inf, 0.25], dtype=torch.float32, device=d)
    cla.check_log_decay(ok_scalar, "scalar")            # -inf reset, l > 0 growth: accepted
    with pytest.raises(ValueError, match="finite and <= 0"):
        cla.check_log_decay(ok_scalar, "gla")           # the same values break the GLA rule
    for bad in (np.nan, np.inf):
        t = torch.tensor([-0.5, bad, -1.0], dtype=torch.float32, device=d)
        with pytest.raises(ValueError):
            cla.check_log_decay(t, "scalar")
    cla.check_log_decay(torch.full((1000,), -0.01, device=d), "gla")

    B, H, T, DK, DV = 1, 2, 200, 64, 64
    g = torch.Generator(device="cpu").manual_seed(11)
    q = (torch.randn(B, H, T, DK, generator=g) / 8).to(torch.bfloat16).to(d)
    k = (torch.randn(B, H, T, DK, generator=g) / 8).to(torch.bfloat16).to(d)
    v = torch.randn(B, H, T, DV, generator=g).to(torch.bfloat16).to(d)
    l = torch.full((B, H, T), -0.05, device=d)
    l[0, 1, 77] = float("nan")
    prev = cla.set_input_checks(True)
    try:
        with pytest.raises(ValueError, match="1 nan"):
            cla.chunked_linear_attn(q, k, v, l)
        lg = torch.full((B, H, T, DK), -0.05, device=d)
        lg[0, 0, 5, 3] = 0.5
        with pytest.raises(ValueError, match="1 positive"):
            cla.gla(q, k, v, lg)
    finally:
        cla.set_input_checks(prev)
    # unchecked, the NaN runs through: in its head every output from that
    # token on is NaN (its decay enters every later cumulative log and the
    # state), the earlier ones and the other head are untouched
    o, _ = cla.chunked_linear_attn(q, k, v, l)
    o = o.float().cpu()
    assert torch.isfinite(o[0, 0]).all()
    assert torch.isfinite(o[0, 1, :77]).all()
    assert torch.isnan(o[0, 1, 77:]).all()

