"""Parity of the HIP chunkwise forward (bf16 in, fp32 state) against the
float64 oracle, through the C ABI (GPU).

Tolerance: relative L2 error <= 2e-2 per output tensor (o, S_T), computed in
float64 against the oracle run on the exact device inputs (bf16 bits and fp32
log decays upcast).
"""

import math

import numpy as np
import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _fwd(ci):
    import chunkwise_linear_attention_amd as cla
    from gpu_util import to_dev
    q, k, v, l, S0 = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0))
    return cla.chunked_linear_attn(q, k, v, l, S0)


def _check_fwd(ci, got, coracle, heads=None):
    from gpu_util import rel_l2, to_np
    o, ST = got
    B, H, T, DK = ci.q.shape
    DV = ci.v.shape[-1]
    o_r, ST_r = coracle.la_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0, heads=heads)
    o_g = to_np(o).reshape(B * H, T, DV)
    ST_g = to_np(ST).reshape(B * H, DK, DV)
    if heads is not None:
        o_g, ST_g = o_g[heads], ST_g[heads]
    e = {"o": rel_l2(o_g, o_r), "ST": rel_l2(ST_g, ST_r)}
    for k_, v_ in e.items():
        assert v_ <= TOL, (k_, v_, e)
    return e


CASES = [
    # (B, H, T, DK, DV, decay, S0, seed)
    (1, 1, 1, 64, 64, "softplus", False, 1),
    (1, 2, 64, 64, 64, "softplus", True, 2),
    (2, 2, 150, 64, 128, "softplus", True, 3),
    (1, 3, 257, 128, 64, "softplus", False, 4),
    (2, 1, 1000, 128, 128, "softplus", True, 5),
    (1, 1, 4096, 64, 64, "softplus", True, 6),      # one head: 16 segments
    (1, 2, 3000, 128, 128, "mix", False, 7),        # strong/weak decay mix, segments
    (3, 5, 700, 128, 64, "head_const", True, 8),
    (2, 2, 200, 64, 64, "zero", True, 9),           # no decay
    # exact resets (l = -inf): sparse, dense, and across segments
    (1, 2, 300, 64, 64, ("resets", 0.02), True, 10),
    (2, 1, 1000, 128, 128, ("resets", 0.05), True, 11),
    (1, 1, 4096, 64, 128, ("resets", 0.003), True, 12),
    (1, 2, 200, 128, 64, ("resets", 0.5), False, 13),
]


@pytest.mark.parametrize("B,H,T,DK,DV,decay,S0,seed", CASES)
def test_chunk_fwd_parity(coracle, B, H, T, DK, DV, decay, S0, seed):
    from gpu_util import say
    say(f"[chunk fwd] B={B} H={H} T={T} DK={DK} DV={DV} decay={decay} S0={S0} seed={seed}")
    ci = syn.chunk_inputs(B, H, T, DK, DV, seed, qk_scale=1 / math.sqrt(DK),
                          decay=decay, S0_scale=0.1 if S0 else None)
    _check_fwd(ci, _fwd(ci), coracle)


def test_chunk_fwd_empty_and_stitched(coracle):
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, rel_l2, say, to_dev, to_np
    say("[chunk fwd] T=0 and two stitched pieces")
    S0 = torch.randn((1, 2, 64, 64), device=dev())
    z = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev())
    o, ST = cla.chunked_linear_attn(z, z, z, torch.zeros((1, 2, 0), device=dev()), S0)
    assert o.shape == (1, 2, 0, 64) and torch.equal(ST, S0)
    ci = syn.chunk_inputs(1, 2, 333, 64, 64, 12, qk_scale=0.125, S0_scale=0.1)
    q, k, v, l, S0 = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0))
    s = 190
    p = lambda x: x[:, :, :s].contiguous()
    r = lambda x: x[:, :, s:].contiguous()
    o1, S1 = cla.chunked_linear_attn(p(q), p(k), p(v), p(l), S0)
    o2, S2 = cla.chunked_linear_attn(r(q), r(k), r(v), r(l), S1)
    o_r, ST_r = coracle.la_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0)
    assert rel_l2(to_np(torch.cat([o1, o2], 2)).reshape(2, 333, 64), o_r) <= TOL
    assert rel_l2(to_np(S2).reshape(2, 64, 64), ST_r) <= TOL


def test_chunk_fwd_deterministic():
    import torch
    from gpu_util import say
    say("[chunk fwd] determinism, B=1 H=2 T=3000 (segmented)")
    ci = syn.chunk_inputs(1, 2, 3000, 128, 64, 13, qk_scale=0.09, S0_scale=0.1)
    o1, S1 = _fwd(ci)
    o2, S2 = _fwd(ci)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_chunk_fwd_resets_at_chunk_edges(coracle):
    """Resets on the first token, on the last token of a chunk and on the
    first of the next, and on two neighbours."""
    from gpu_util import say
    say("[chunk fwd] resets at chunk edges")
    ci = syn.chunk_inputs(1, 2, 260, 64, 64, 31, qk_scale=1 / 8, S0_scale=0.1)
    ci.l[0, 0, [0, 63, 64, 127, 128]] = -np.inf
    ci.l[0, 1, [191, 192, 259]] = -np.inf
    _check_fwd(ci, _fwd(ci), coracle)
