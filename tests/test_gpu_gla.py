"""Parity of the HIP kernels with one decay per key dimension (gated linear
attention) against the float64 oracle, through the C ABI (GPU).

Tolerance: relative L2 error <= 2e-2 per output tensor, computed in float64
against the oracle run on the exact device inputs (bf16 bits and fp32 log
decays upcast).
"""

import numpy as np
import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _gla_fwd(ci):
    import chunkwise_linear_attention_amd as cla
    from gpu_util import to_dev
    q, k, v, l, S0 = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0))
    return cla.gla(q, k, v, l, S0)


def _check_fwd(ci, got, coracle, heads=None):
    from gpu_util import rel_l2, to_np
    o, ST = got
    B, H, T, DK = ci.q.shape
    DV = ci.v.shape[-1]
    o_r, ST_r = coracle.gla_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0, heads=heads)
    o_g = to_np(o).reshape(B * H, T, DV)
    ST_g = to_np(ST).reshape(B * H, DK, DV)
    if heads is not None:
        o_g, ST_g = o_g[heads], ST_g[heads]
    e = {"o": rel_l2(o_g, o_r), "ST": rel_l2(ST_g, ST_r)}
    for k_, v_ in e.items():
        assert v_ <= TOL, (k_, v_, e)
    return e


FWD_CASES = [
    # (B, H, T, DK, DV, decay, S0, seed)
    (1, 1, 1, 64, 64, "logsigmoid", False, 1),
    (1, 2, 64, 64, 64, "logsigmoid", True, 2),
    (2, 2, 150, 64, 128, "logsigmoid", True, 3),
    (1, 3, 257, 128, 64, ("uniform", -1.0, 0.0), False, 4),
    (2, 1, 1000, 128, 128, "logsigmoid", True, 5),
    (1, 2, 700, 128, 128, ("logsigmoid", 1.0), True, 6),     # stronger gates
    (1, 2, 300, 64, 64, ("uniform", -8.0, 0.0), True, 7),    # blocks past exp(-60): exact path
    (1, 1, 200, 128, 128, ("const", -5.0), True, 8),         # every block exact
    (2, 2, 333, 128, 64, ("uniform", -0.02, 0.0), True, 9),  # weak decays
    (1, 2, 130, 64, 128, ("const", 0.0), False, 10),         # no decay
    # few sequence-heads, long sequences: split into segments of 16-chunk blocks
    (1, 2, 3000, 64, 64, "logsigmoid", True, 11),            # 3 segments
    (1, 1, 5000, 128, 128, ("uniform", -0.05, 0.0), True, 12),  # 5 segments, weak decays
    (2, 1, 2100, 128, 64, ("logsigmoid", 1.0), False, 13),   # ragged last segment
    (1, 1, 4200, 64, 64, ("uniform", -8.0, 0.0), True, 14),  # exact blocks across segments
]


@pytest.mark.parametrize("B,H,T,DK,DV,decay,S0,seed", FWD_CASES)
def test_gla_fwd_parity(coracle, B, H, T, DK, DV, decay, S0, seed):
    from gpu_util import say
    say(f"[gla fwd] B={B} H={H} T={T} DK={DK} DV={DV} decay={decay} S0={S0} seed={seed}")
    ci = syn.gla_inputs(B, H, T, DK, DV, seed, decay=decay, S0_scale=0.1 if S0 else None)
    e = _check_fwd(ci, _gla_fwd(ci), coracle)
    say("[gla fwd] rel-L2 " + ", ".join(f"{k}={v:.2e}" for k, v in e.items()))


def test_gla_fwd_empty_and_stitched(coracle):
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, rel_l2, say, to_dev, to_np
    say("[gla fwd] T=0 and two stitched pieces")
    S0 = torch.randn((1, 2, 64, 64), device=dev())
    z = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev())
    o, ST = cla.gla(z, z, z, torch.zeros((1, 2, 0, 64), device=dev()), S0)
    assert o.shape == (1, 2, 0, 64) and torch.equal(ST, S0)
    ci = syn.gla_inputs(1, 2, 333, 64, 64, 12, S0_scale=0.1)
    q, k, v, l, S0 = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0))
    s = 190
    p = lambda x: x[:, :, :s].contiguous()
    r = lambda x: x[:, :, s:].contiguous()
    o1, S1 = cla.gla(p(q), p(k), p(v), p(l), S0)
    o2, S2 = cla.gla(r(q), r(k), r(v), r(l), S1)
    o_r, ST_r = coracle.gla_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0)
    assert rel_l2(to_np(torch.cat([o1, o2], 2)).reshape(2, 333, 64), o_r) <= TOL
    assert rel_l2(to_np(S2).reshape(2, 64, 64), ST_r) <= TOL


def test_gla_fwd_equal_decays_match_scalar_kernel():
    """With the same log decay in every key dimension the vector kernel and
    the scalar one compute the same recurrence."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import rel_l2, say, to_dev, to_np
    say("[gla fwd] equal decays vs the scalar kernel")
    ci = syn.chunk_inputs(2, 2, 500, 128, 64, 77, qk_scale=1 / np.sqrt(128), S0_scale=0.1)
    lv = np.repeat(ci.l[..., None], 128, axis=-1).copy()
    q, k, v, l, lvd, S0 = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, lv, ci.S0))
    o_s, S_s = cla.chunked_linear_attn(q, k, v, l, S0)
    o_v, S_v = cla.gla(q, k, v, lvd, S0)
    torch.cuda.synchronize()
    assert rel_l2(to_np(o_v), to_np(o_s).astype(np.float64)) <= 1e-2
    assert rel_l2(to_np(S_v), to_np(S_s).astype(np.float64)) <= 1e-2


def test_gla_fwd_deterministic():
    import torch
    from gpu_util import say
    say("[gla fwd] determinism")
    ci = syn.gla_inputs(1, 2, 900, 128, 128, 13, S0_scale=0.1)
    o1, S1 = _gla_fwd(ci)
    o2, S2 = _gla_fwd(ci)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


BWD_NAMES = ("dq", "dk", "dv", "dl", "dS0")

BWD_CASES = [
    # (B, H, T, DK, DV, decay, S0, dST, seed)
    (1, 1, 1, 64, 64, "logsigmoid", False, False, 21),
    (1, 2, 64, 64, 64, "logsigmoid", True, True, 22),
    (2, 2, 150, 64, 128, "logsigmoid", True, True, 23),
    (1, 3, 257, 128, 64, ("uniform", -1.0, 0.0), False, False, 24),
    (2, 1, 1000, 128, 128, "logsigmoid", True, True, 25),
    (1, 1, 2500, 64, 64, "logsigmoid", True, True, 26),       # 3 segments of 16 chunks
    (1, 2, 4100, 128, 128, ("uniform", -0.05, 0.0), True, True, 27),  # 5 segments, weak decays
    (1, 2, 300, 64, 64, ("uniform", -8.0, 0.0), True, True, 28),     # exact paths
    (1, 1, 200, 128, 128, ("const", -5.0), True, True, 29),          # every block exact
    (1, 2, 700, 128, 128, ("logsigmoid", 1.0), True, False, 30),
    (1, 2, 130, 64, 128, ("const", 0.0), False, True, 31),           # no decay
    # few sequence-heads, long sequences: split into segments of 16-chunk blocks
    (1, 2, 16384, 128, 128, "logsigmoid", True, True, 32),            # 16 segments
    (1, 1, 4200, 64, 64, ("uniform", -8.0, 0.0), True, True, 33),     # exact blocks, 5 segments
    (2, 1, 2100, 128, 64, ("logsigmoid", 1.0), False, True, 34),      # ragged last segment
]


def _gla_bwd(ci):
    import chunkwise_linear_attention_amd as cla
    from gpu_util import to_dev
    q, k, v, l, S0, dO, dST = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    return cla.gla_bwd(q, k, v, l, S0, dO, dST)


def _check_bwd(ci, got, coracle, heads=None):
    from gpu_util import rel_l2, to_np
    B, H = ci.q.shape[:2]
    ref = coracle.gla_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST, heads=heads)
    errs = {}
    for name, g, r in zip(BWD_NAMES, got, ref):
        gn = to_np(g).reshape(B * H, *r.shape[1:])
        if heads is not None:
            gn = gn[heads]
        errs[name] = rel_l2(gn, r)
    for k_, v_ in errs.items():
        assert v_ <= TOL, (k_, v_, errs)
    return errs


@pytest.mark.parametrize("B,H,T,DK,DV,decay,S0,dST,seed", BWD_CASES)
def test_gla_bwd_parity(coracle, B, H, T, DK, DV, decay, S0, dST, seed):
    from gpu_util import say
    say(f"[gla bwd] B={B} H={H} T={T} DK={DK} DV={DV} decay={decay} S0={S0} dST={dST}")
    ci = syn.gla_inputs(B, H, T, DK, DV, seed, decay=decay, S0_scale=0.1 if S0 else None,
                        dST_scale=0.1 if dST else None)
    errs = _check_bwd(ci, _gla_bwd(ci), coracle)
    say("[gla bwd] rel-L2 " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_gla_bwd_empty_and_deterministic():
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, say
    say("[gla bwd] T=0 and determinism")
    dST = torch.randn((1, 2, 64, 64), device=dev())
    z = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev())
    lz = torch.zeros((1, 2, 0, 64), device=dev())
    g = cla.gla_bwd(z, z, z, lz, None, z, dST)
    assert torch.equal(g[4], dST)
    ci = syn.gla_inputs(1, 2, 1200, 128, 64, 33, S0_scale=0.1, dST_scale=0.1)
    a = _gla_bwd(ci)
    b = _gla_bwd(ci)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_gla_bwd_equal_decays_match_scalar_kernel():
    """Equal decays in every key dimension: dq, dk, dv, dS0 equal the scalar
    kernel's, and the vector decay gradient sums to the scalar one."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import rel_l2, say, to_dev, to_np
    say("[gla bwd] equal decays vs the scalar kernel")
    ci = syn.chunk_inputs(1, 2, 700, 64, 64, 78, qk_scale=1 / 8, S0_scale=0.1, dST_scale=0.1)
    lv = np.repeat(ci.l[..., None], 64, axis=-1).copy()
    q, k, v, l, lvd, S0, dO, dST = (to_dev(x) for x in
                                    (ci.q, ci.k, ci.v, ci.l, lv, ci.S0, ci.dO, ci.dST))
    gs = cla.chunked_linear_attn_bwd(q, k, v, l, S0, dO, dST)
    gv = cla.gla_bwd(q, k, v, lvd, S0, dO, dST)
    torch.cuda.synchronize()
    for i in (0, 1, 2, 4):
        assert rel_l2(to_np(gv[i]), to_np(gs[i])) <= 1e-2, i
    assert rel_l2(to_np(gv[3]).sum(-1), to_np(gs[3])) <= 2e-2


@pytest.mark.parametrize("variant", ["plain", "S0_dST"])
def test_gla_workload_sampled_heads(coracle, variant):
    """The bench's GLA workload (B=32, H=16, T=4096, dk=dv=128) at full size, in
    the launch configuration the bench times, against the oracle on sampled
    sequences (the whole tensors and every 1024-token block of each);
    every output finite.  The second variant adds S0 and dS_T."""
    import torch
    from gpu_util import CHUNK_BLOCKS, block_rel_l2, rel_l2, say, to_np
    if variant == "plain":
        ci = syn.WORKLOADS["gla_T4096"].make()
    else:
        ci = syn.gla_inputs(32, 16, 4096, 128, 128, 1061, S0_scale=0.1, dST_scale=0.1)
    B, H = ci.q.shape[:2]
    heads = np.array(sorted({0, (B * H) // 2 + 1, B * H - 1}), dtype=np.int64)
    say(f"[gla workload] {variant} shape={ci.q.shape} heads={heads.tolist()}")
    o, ST = _gla_fwd(ci)
    g = _gla_bwd(ci)
    torch.cuda.synchronize()
    out = (o, ST) + tuple(g)
    names = ("o", "ST") + BWD_NAMES
    for name, t in zip(names, out):
        assert bool(torch.isfinite(t.float()).all()), name
    o_r, ST_r = coracle.gla_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0, heads=heads)
    refs = (o_r, ST_r) + tuple(coracle.gla_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST,
                                               heads=heads))
    errs = {}
    for name, t, r in zip(names, out, refs):
        if t is None:
            continue
        got = to_np(t.reshape(B * H, *t.shape[2:])[torch.from_numpy(heads).to(t.device)])
        got = got.reshape(r.shape)
        errs[name] = rel_l2(got, r)
        errs[name + "_blk"] = block_rel_l2(got, r, CHUNK_BLOCKS[name])[0]
    say(f"[gla workload] {variant} rel-L2: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, errs


@pytest.mark.parametrize("B,H,T,DK,DV,S0,dST,seed", [
    (1, 2, 4100, 128, 128, True, True, 41),    # 5 segments
    (1, 1, 3000, 64, 64, False, True, 42),     # 3 segments, ragged tail
    (2, 1, 200, 64, 128, True, False, 43),     # not split: nothing saved
])
def test_gla_saved_states_bit_identical(B, H, T, DK, DV, S0, dST, seed):
    """cla_gla_fwd_saved then cla_gla_bwd_saved (the backward's segments start
    from the forward's saved states) give exactly the outputs of the plain
    calls, which rerun the state pass."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import say, to_dev
    say(f"[gla saved] B={B} H={H} T={T} DK={DK} DV={DV} S0={S0} dST={dST}")
    gi = syn.gla_inputs(B, H, T, DK, DV, seed, S0_scale=0.1 if S0 else None,
                        dST_scale=0.1 if dST else None)
    q, k, v, l, S0d, dO, dSTd = (to_dev(x) for x in (gi.q, gi.k, gi.v, gi.l, gi.S0, gi.dO, gi.dST))
    o1, ST1 = cla.gla(q, k, v, l, S0d)
    g1 = cla.gla_bwd(q, k, v, l, S0d, dO, dSTd)
    o2, ST2, saved = cla.gla(q, k, v, l, S0d, save_states=True)
    assert saved.numel() == max(1, cla.gla_saved_bytes(B, H, T, DK, DV))
    g2 = cla.gla_bwd(q, k, v, l, S0d, dO, dSTd, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ST1, ST2)
    for x, y in zip(g1, g2):
        assert (x is None and y is None) or torch.equal(x, y)


def test_gla_long_workload_full_heads(coracle):
    """The long GLA workload (B=1, H=16, T=98304: 32 segments) at full size,
    through the saved-state path the bench times, against the oracle on two
    whole sequence-heads: every output (o, S_T, dq, dk, dv, dl, dS0), the
    whole tensors and every 1024-token block.  The plain calls give
    bit-identical results; every output is finite."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import CHUNK_BLOCKS, block_rel_l2, rel_l2, say, to_dev, to_np
    ci = syn.WORKLOADS["gla_long_T98304"].make()
    B, H, T, DK = ci.q.shape
    heads = np.array([0, 9], dtype=np.int64)
    say(f"[gla long workload] shape={ci.q.shape} heads={heads.tolist()}")
    q, k, v, l, dO = (to_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.dO))
    o, ST, saved = cla.gla(q, k, v, l, None, save_states=True)
    g = cla.gla_bwd(q, k, v, l, None, dO, None, saved=saved)
    o2, ST2 = cla.gla(q, k, v, l, None)
    g2 = cla.gla_bwd(q, k, v, l, None, dO, None)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ST, ST2)
    for x, y in zip(g, g2):
        assert (x is None and y is None) or torch.equal(x, y)
    out = (o, ST) + tuple(g)
    names = ("o", "ST", "dq", "dk", "dv", "dl", "dS0")
    for name, t in zip(names, out):
        assert bool(torch.isfinite(t.float()).all()), name
    say("[gla long workload] oracle on two whole heads")
    o_r, ST_r = coracle.gla_fwd(ci.q, ci.k, ci.v, ci.l, None, heads=heads)
    refs = (o_r, ST_r) + tuple(coracle.gla_bwd(ci.q, ci.k, ci.v, ci.l, None, ci.dO, None,
                                               heads=heads))
    hsel = torch.from_numpy(heads)
    errs = {}
    for name, t, r in zip(names, out, refs):
        got = to_np(t.reshape(B * H, *t.shape[2:])[hsel.to(t.device)]).reshape(r.shape)
        errs[name] = rel_l2(got, r)
        errs[name + "_blk"] = block_rel_l2(got, r, CHUNK_BLOCKS[name])[0]
    say("[gla long workload] rel-L2 " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
    assert all(v_ <= TOL for v_ in errs.values()), errs
