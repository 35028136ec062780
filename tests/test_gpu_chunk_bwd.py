"""Parity of the HIP chunkwise backward (dq, dk, dv, dlog_decay, dS0) against
the float64 oracle's adjoint recurrence, through the C ABI (GPU).

Tolerance: relative L2 error <= 2e-2 per output tensor, computed in float64
against the oracle run on the exact device inputs.
"""

import math

import numpy as np
import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu
TOL = 2e-2
NAMES = ("dq", "dk", "dv", "dl", "dS0")


def _bwd(ci):
    import chunkwise_linear_attention_amd as cla
    from gpu_util import to_dev
    q, k, v, l, S0, dO, dST = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    return cla.chunked_linear_attn_bwd(q, k, v, l, S0, dO, dST)


def _check_bwd(ci, got, coracle):
    from gpu_util import rel_l2, to_np
    B, H, T, DK = ci.q.shape
    ref = coracle.la_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST)
    errs = {}
    for name, g, r in zip(NAMES, got, ref):
        errs[name] = rel_l2(to_np(g).reshape(r.shape), r)
    for k_, v_ in errs.items():
        assert v_ <= TOL, (k_, v_, errs)
    return errs


CASES = [
    # (B, H, T, DK, DV, decay, S0, dST, seed)
    (1, 1, 1, 64, 64, "softplus", False, False, 1),
    (1, 2, 64, 64, 64, "softplus", True, True, 2),
    (2, 2, 150, 64, 128, "softplus", True, True, 3),
    (1, 3, 257, 128, 64, "softplus", False, False, 4),
    (2, 1, 1000, 128, 128, "softplus", True, True, 5),
    (1, 1, 4096, 64, 64, "softplus", True, True, 6),       # 16 segments
    (1, 2, 3000, 128, 128, "mix", False, True, 7),          # strong/weak decays, segments
    (3, 5, 700, 128, 64, "head_const", True, False, 8),
    (2, 2, 200, 64, 64, "zero", True, True, 9),
    # exact resets (l = -inf)
    (1, 2, 300, 64, 64, ("resets", 0.02), True, True, 10),
    (2, 1, 1000, 128, 128, ("resets", 0.05), True, True, 11),
    (1, 1, 4096, 64, 128, ("resets", 0.003), True, False, 12),
    (1, 2, 200, 128, 64, ("resets", 0.5), False, True, 13),
]


@pytest.mark.parametrize("B,H,T,DK,DV,decay,S0,dST,seed", CASES)
def test_chunk_bwd_parity(coracle, B, H, T, DK, DV, decay, S0, dST, seed):
    from gpu_util import say
    say(f"[chunk bwd] B={B} H={H} T={T} DK={DK} DV={DV} decay={decay} S0={S0} dST={dST} seed={seed}")
    ci = syn.chunk_inputs(B, H, T, DK, DV, seed, qk_scale=1 / math.sqrt(DK), decay=decay,
                          S0_scale=0.1 if S0 else None, dST_scale=0.1 if dST else None)
    _check_bwd(ci, _bwd(ci), coracle)


SAVED_CASES = [
    # sequences split into backward segments (few heads), ragged ends
    (1, 2, 2500, 64, 64, "softplus", True, True, 21),
    (1, 1, 3001, 128, 128, "mix", True, False, 22),
    (2, 1, 1100, 128, 64, "softplus", False, True, 23),
    (1, 1, 700, 64, 128, "head_const", True, True, 24),
    (1, 4, 100, 64, 64, "softplus", True, True, 25),   # one segment: nothing saved
    (1, 1, 2600, 128, 128, ("resets", 0.01), True, True, 26),
]


@pytest.mark.parametrize("B,H,T,DK,DV,decay,S0,dST,seed", SAVED_CASES)
def test_chunk_saved_states_parity(coracle, B, H, T, DK, DV, decay, S0, dST, seed):
    """cla_chunk_fwd_saved then cla_chunk_bwd_saved: the backward starts its
    segments from the forward's states; every output against the oracle."""
    import chunkwise_linear_attention_amd as cla
    from gpu_util import rel_l2, say, to_dev, to_np
    say(f"[chunk saved] B={B} H={H} T={T} DK={DK} DV={DV} decay={decay} S0={S0} dST={dST}")
    ci = syn.chunk_inputs(B, H, T, DK, DV, seed, qk_scale=1 / math.sqrt(DK), decay=decay,
                          S0_scale=0.1 if S0 else None, dST_scale=0.1 if dST else None)
    q, k, v, l, S0d, dO, dSTd = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    o, ST, saved = cla.chunked_linear_attn(q, k, v, l, S0d, save_states=True)
    assert saved.numel() == max(1, cla.chunk_saved_bytes(B, H, T, DK, DV))
    o_r, ST_r = coracle.la_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0)
    assert rel_l2(to_np(o).reshape(o_r.shape), o_r) <= TOL
    assert rel_l2(to_np(ST).reshape(ST_r.shape), ST_r) <= TOL
    got = cla.chunked_linear_attn_bwd(q, k, v, l, S0d, dO, dSTd, saved=saved)
    errs = _check_bwd(ci, got, coracle)
    say(f"[chunk saved] rel-L2 " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))


def test_chunk_bwd_empty_sequence():
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, say
    say("[chunk bwd] T=0")
    z = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev())
    l = torch.zeros((1, 2, 0), device=dev())
    dST = torch.randn((1, 2, 64, 64), device=dev())
    dq, dk, dv, dl, dS0 = cla.chunked_linear_attn_bwd(z, z, z, l, None, z, dST)
    assert dq.shape == (1, 2, 0, 64) and dl.shape == (1, 2, 0)
    assert torch.equal(dS0, dST)


def test_chunk_bwd_stitched_pieces(coracle):
    """Two pieces: the second starts from the first's final state; the first's
    backward receives the second's dS0 as its final-state gradient."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import rel_l2, say, to_dev, to_np
    say("[chunk bwd] stitched pieces T=190+143, DK=128 DV=64")
    ci = syn.chunk_inputs(1, 2, 333, 128, 64, 21, qk_scale=1 / math.sqrt(128),
                          S0_scale=0.1, dST_scale=0.1)
    q, k, v, l, S0, dO, dST = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    s = 190
    p = lambda x: x[:, :, :s].contiguous()
    r = lambda x: x[:, :, s:].contiguous()
    _, S1 = cla.chunked_linear_attn(p(q), p(k), p(v), p(l), S0)
    g2 = cla.chunked_linear_attn_bwd(r(q), r(k), r(v), r(l), S1, r(dO), dST)
    g1 = cla.chunked_linear_attn_bwd(p(q), p(k), p(v), p(l), S0, p(dO), g2[4])
    ref = coracle.la_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST)
    for i in range(4):
        got = to_np(torch.cat([g1[i], g2[i]], 2)).reshape(ref[i].shape)
        assert rel_l2(got, ref[i]) <= TOL, NAMES[i]
    assert rel_l2(to_np(g1[4]).reshape(ref[4].shape), ref[4]) <= TOL


def test_chunk_bwd_deterministic():
    import torch
    from gpu_util import say
    say("[chunk bwd] determinism, B=1 H=2 T=3000 (segmented)")
    ci = syn.chunk_inputs(1, 2, 3000, 128, 64, 23, qk_scale=0.09, S0_scale=0.1, dST_scale=0.1)
    a = _bwd(ci)
    b = _bwd(ci)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_chunk_unaligned_state_pointers(coracle):
    """fp32 state tensors need only 4-byte alignment: S0 and dS_T at an odd
    float offset, read directly and transposed (dQ pass), segments present."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, say, to_dev
    say("[chunk bwd] unaligned S0 / dST")
    B, H, T, DK, DV = 1, 2, 1500, 128, 64
    ci = syn.chunk_inputs(B, H, T, DK, DV, 41, qk_scale=1 / math.sqrt(DK), S0_scale=0.1,
                          dST_scale=0.1)
    n = B * H * DK * DV

    def odd(x):
        buf = torch.zeros(n + 1, dtype=torch.float32, device=dev())
        buf[1:] = torch.from_numpy(x.reshape(-1)).to(dev())
        return buf[1:].view(B, H, DK, DV)

    q, k, v, l, dO = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.dO))
    S0, dST = odd(ci.S0), odd(ci.dST)
    assert S0.data_ptr() % 16 == 4
    o, ST, saved = cla.chunked_linear_attn(q, k, v, l, S0, save_states=True)
    _check_bwd(ci, cla.chunked_linear_attn_bwd(q, k, v, l, S0, dO, dST), coracle)
    _check_bwd(ci, cla.chunked_linear_attn_bwd(q, k, v, l, S0, dO, dST, saved=saved), coracle)
