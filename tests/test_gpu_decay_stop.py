"""Sequences whose decay product reaches exactly 0 in fp32 partway through a
segment (GPU).

A segment's state from a zero start is a sum of chunk contributions, each
scaled by the decay from its chunk to the segment's end; the forward's segment
pass adds them last to first and stops once that running product is 0, and
the dQ pass stops adding to a segment's local state gradient once the decay
from the segment start is 0.  Here a constant log decay makes the product
vanish after a known number of chunks, inside the segments of both passes;
every output is compared with the float64 oracle on sampled sequences (the
whole tensors and every 1024-token block of each), through the saved-state
path and the plain calls.
"""

import math

import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu
TOL = 2e-2
NAMES = ("o", "ST", "dq", "dk", "dv", "dl", "dS0")

CASES = [
    # (B, H, T, DK, DV, l, seed) with the chunk decay exp(64 l) reaching 0 in
    # fp32 after about 103 / (64 |l|) chunks
    (4, 32, 5120, 64, 64, -0.1, 41),      # forward segments of 20 chunks: stop after ~17
    (2, 64, 10240, 128, 128, -0.05, 42),  # forward segments of 40 chunks: stop after ~33
    (1, 16, 16384, 64, 64, -0.2, 43),     # backward segments of 16 chunks: G sums stop after ~8
    (1, 16, 16384, 128, 64, -0.11, 44),   # backward segments of 16 chunks: stop after ~15
]


def _run(ci, saved):
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import to_dev
    q, k, v, l, S0, dO, dST = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    if saved:
        o, ST, sv = cla.chunked_linear_attn(q, k, v, l, S0, save_states=True)
        g = cla.chunked_linear_attn_bwd(q, k, v, l, S0, dO, dST, saved=sv)
    else:
        o, ST = cla.chunked_linear_attn(q, k, v, l, S0)
        g = cla.chunked_linear_attn_bwd(q, k, v, l, S0, dO, dST)
    torch.cuda.synchronize()
    return (o, ST) + tuple(g)


@pytest.mark.parametrize("saved", [True, False], ids=["saved", "recomputed"])
@pytest.mark.parametrize("B,H,T,DK,DV,lval,seed", CASES)
def test_decay_product_reaches_zero(coracle, B, H, T, DK, DV, lval, seed, saved):
    import torch
    from gpu_util import CHUNK_BLOCKS, block_rel_l2, rel_l2, say, to_np
    say(f"[decay stop] B={B} H={H} T={T} DK={DK} DV={DV} l={lval} saved={saved}")
    ci = syn.chunk_inputs(B, H, T, DK, DV, seed, qk_scale=1 / math.sqrt(DK),
                          decay=("const", lval), S0_scale=0.1, dST_scale=0.1)
    out = _run(ci, saved)
    for name, t in zip(NAMES, out):
        assert bool(torch.isfinite(t.float()).all()), name
    nh = B * H
    heads = sorted({0, nh // 2 + 1, nh - 1})
    o_r, ST_r = coracle.la_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0, heads=heads)
    g_r = coracle.la_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST, heads=heads)
    errs = {}
    for name, t, r in zip(NAMES, out, (o_r, ST_r) + tuple(g_r)):
        got = to_np(t.reshape(nh, *t.shape[2:])[heads]).reshape(r.shape)
        errs[name] = rel_l2(got, r)
        errs[name + "_blk"] = block_rel_l2(got, r, CHUNK_BLOCKS[name])[0]
    say("[decay stop] rel-L2 " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, errs
