"""Tensors past 2^31 elements (GPU): every kernel's element offsets leave the
int32 range, so a 32-bit index anywhere on the path would read or write the
wrong element.  Device tensors are filled with seeded filler of the same
distributions; the sampled channels (scan) or sequence-heads (chunkwise) are
overwritten with the seeded inputs of the synthetic generators, which the
oracle also reads, so that the compared outputs depend on those inputs only
(channels and heads are independent).  The sampled ones include the last
channels of the last batch row (offsets above 2^31 in the last steps) and
the last head (every offset above 2^31).

Bars as elsewhere: scan relative L2 <= 1e-5, chunkwise <= 2e-2, for each
whole sampled tensor and every block (1024 steps of one channel; 1024
tokens of one head); every output finite everywhere.
"""

import math

import numpy as np
import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu


def _check(name, got, ref, blocks, tol, errs):
    from gpu_util import block_rel_l2, rel_l2
    errs[name] = rel_l2(got, ref)
    errs[name + "_blk"], at = block_rel_l2(got, ref, blocks)
    assert errs[name] <= tol, (name, errs[name])
    assert errs[name + "_blk"] <= tol, (name, "block", at, errs[name + "_blk"])


def test_scan_past_int32_elements(coracle):
    """B=2, T=2^20+37, D=1024 (2,147,559,424 elements per tensor): the XCD
    order, the time split into 16 segments and the ragged last block, on 7
    sampled channels of both batch rows."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, say
    B, T, D = 2, (1 << 20) + 37, 1024
    assert B * T * D > 2 ** 31
    sel = np.array([0, 1, 63, 64, 511, 1022, 1023], dtype=np.int64)
    say(f"[scan maxsize] B={B} T={T} D={D} channels={sel.tolist()}")
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(2031)
    a = torch.empty(B, T, D, device=d).uniform_(1e-4, 0.5, generator=g).neg_().exp_()
    b = torch.randn(B, T, D, device=d, generator=g)
    dh = torch.randn(B, T, D, device=d, generator=g)
    h0 = torch.randn(B, D, device=d, generator=g)
    dhT = torch.randn(B, D, device=d, generator=g)
    inp = syn.scan_inputs(B, T, len(sel), 2031, delta=(1e-4, 0.5), h0=True, dhT=True)
    idx = torch.from_numpy(sel).to(d)
    for x, v in ((a, inp.a), (b, inp.b), (dh, inp.dh)):
        x.index_copy_(2, idx, torch.from_numpy(v).to(d))
    for x, v in ((h0, inp.h0), (dhT, inp.dhT)):
        x.index_copy_(1, idx, torch.from_numpy(v).to(d))
    h, hT = cla.scan(a, b, h0)
    da, db, dh0 = cla.scan_bwd(a, h, h0, dh, dhT)
    torch.cuda.synchronize()
    for name, t in (("h", h), ("hT", hT), ("da", da), ("db", db), ("dh0", dh0)):
        assert bool(torch.isfinite(t).all()), name
    got = {"h": h.index_select(2, idx), "da": da.index_select(2, idx),
           "db": db.index_select(2, idx), "hT": hT.index_select(1, idx),
           "dh0": dh0.index_select(1, idx)}
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in got.items()}
    del a, b, dh, h, da, db
    torch.cuda.empty_cache()
    say("[scan maxsize] oracle on the sampled channels")
    hr, hTr = coracle.scan_fwd(inp.a, inp.b, inp.h0)
    dar, dbr, dh0r = coracle.scan_bwd(inp.a, hr.astype(np.float32), inp.h0, inp.dh, inp.dhT)
    errs = {}
    for name, ref, blk in (("h", hr, (1, 1024, 1)), ("da", dar, (1, 1024, 1)),
                           ("db", dbr, (1, 1024, 1)), ("hT", hTr, (1, 1)),
                           ("dh0", dh0r, (1, 1))):
        _check(name, got[name], ref, blk, 1e-5, errs)
    # the steps of the last batch row whose offsets are past 2^31 elements,
    # scored together (a single element near zero has no meaningful relative
    # error)
    t_hi = (2 ** 31 - (B - 1) * T * D) // D
    for name, ref in (("h", hr), ("da", dar), ("db", dbr)):
        _check(name + "_tail", got[name][B - 1, t_hi:], ref[B - 1, t_hi:], (), 1e-5, errs)
    say("[scan maxsize] rel-L2: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))


def test_chunk_past_int32_elements(coracle):
    """B=1, H=257, T=65536, dk=dv=128 (2,155,872,256 elements per q, k, dq,
    dk tensor), decays -1e-5 / -5 mixed, S0 and dS_T given, through the
    saved-state training path; the oracle on heads 0, 128 and 256 (head 256
    starts at element 2^31)."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import CHUNK_BLOCKS, dev, say, to_dev, to_np
    B, H, T, DK, DV = 1, 257, 65536, 128, 128
    assert B * H * T * DK > 2 ** 31
    heads = np.array([0, 128, 256], dtype=np.int64)
    say(f"[chunk maxsize] B={B} H={H} T={T} DK={DK} DV={DV} heads={heads.tolist()}")
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(2032)
    s = 1 / math.sqrt(DK)
    bf = torch.bfloat16
    q = (torch.randn(B, H, T, DK, device=d, generator=g) * s).to(bf)
    k = (torch.randn(B, H, T, DK, device=d, generator=g) * s).to(bf)
    v = torch.randn(B, H, T, DV, device=d, generator=g).to(bf)
    dO = torch.randn(B, H, T, DV, device=d, generator=g).to(bf)
    coin = torch.rand(B, H, T, device=d, generator=g) < 0.5
    l = torch.where(coin, torch.tensor(-5.0, device=d), torch.tensor(-1e-5, device=d))
    S0 = torch.randn(B, H, DK, DV, device=d, generator=g) * 0.1
    dST = torch.randn(B, H, DK, DV, device=d, generator=g) * 0.1
    ci = syn.chunk_inputs(B, len(heads), T, DK, DV, 2032, qk_scale=s, decay="mix",
                          S0_scale=0.1, dST_scale=0.1)
    idx = torch.from_numpy(heads).to(d)
    for x, val in ((q, ci.q), (k, ci.k), (v, ci.v), (dO, ci.dO), (l, ci.l), (S0, ci.S0),
                   (dST, ci.dST)):
        x.index_copy_(1, idx, to_dev(val))
    o, ST, saved = cla.chunked_linear_attn(q, k, v, l, S0, save_states=True)
    gr = cla.chunked_linear_attn_bwd(q, k, v, l, S0, dO, dST, saved=saved)
    torch.cuda.synchronize()
    names = ("o", "ST", "dq", "dk", "dv", "dl", "dS0")
    out = (o, ST) + tuple(gr)
    for name, t in zip(names, out):
        assert bool(torch.isfinite(t.float() if t.dtype == bf else t).all()), name
    got = {n: to_np(t.index_select(1, idx))[0] for n, t in zip(names, out)}
    del q, k, v, dO, o, gr, out, saved
    torch.cuda.empty_cache()
    say("[chunk maxsize] oracle on the sampled heads")
    o_r, ST_r = coracle.la_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0)
    refs = (o_r, ST_r) + tuple(coracle.la_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    errs = {}
    for name, ref in zip(names, refs):
        _check(name, got[name], ref, CHUNK_BLOCKS[name], 2e-2, errs)
    say("[chunk maxsize] rel-L2: " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))


def test_gla_past_int32_elements(coracle):
    """One decay per key dimension at B=1, H=257, T=65536, dk=dv=128 (q, k,
    the log decays, dq, dk and dl past 2^31 elements), S0 and dS_T given,
    through the saved-state training path; the oracle on heads 0, 128 and
    256."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import CHUNK_BLOCKS, dev, say, to_dev, to_np
    B, H, T, DK, DV = 1, 257, 65536, 128, 128
    assert B * H * T * DK > 2 ** 31
    heads = np.array([0, 128, 256], dtype=np.int64)
    say(f"[gla maxsize] B={B} H={H} T={T} DK={DK} DV={DV} heads={heads.tolist()}")
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(2033)
    s = 1 / math.sqrt(DK)
    bf = torch.bfloat16
    q = (torch.randn(B, H, T, DK, device=d, generator=g) * s).to(bf)
    k = (torch.randn(B, H, T, DK, device=d, generator=g) * s).to(bf)
    v = torch.randn(B, H, T, DV, device=d, generator=g).to(bf)
    dO = torch.randn(B, H, T, DV, device=d, generator=g).to(bf)
    l = torch.randn(B, H, T, DK, device=d, generator=g)
    l = torch.nn.functional.logsigmoid(l).div_(16.0)
    S0 = torch.randn(B, H, DK, DV, device=d, generator=g) * 0.1
    dST = torch.randn(B, H, DK, DV, device=d, generator=g) * 0.1
    ci = syn.gla_inputs(B, len(heads), T, DK, DV, 2033, S0_scale=0.1, dST_scale=0.1)
    idx = torch.from_numpy(heads).to(d)
    for x, val in ((q, ci.q), (k, ci.k), (v, ci.v), (dO, ci.dO), (l, ci.l), (S0, ci.S0),
                   (dST, ci.dST)):
        x.index_copy_(1, idx, to_dev(val))
    o, ST, saved = cla.gla(q, k, v, l, S0, save_states=True)
    gr = cla.gla_bwd(q, k, v, l, S0, dO, dST, saved=saved)
    torch.cuda.synchronize()
    names = ("o", "ST", "dq", "dk", "dv", "dl", "dS0")
    out = (o, ST) + tuple(gr)
    for name, t in zip(names, out):
        assert bool(torch.isfinite(t.float() if t.dtype == bf else t).all()), name
    got = {n: to_np(t.index_select(1, idx))[0] for n, t in zip(names, out)}
    del q, k, v, dO, l, o, gr, out, saved
    torch.cuda.empty_cache()
    say("[gla maxsize] oracle on the sampled heads")
    o_r, ST_r = coracle.gla_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0)
    refs = (o_r, ST_r) + tuple(coracle.gla_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    errs = {}
    for name, ref in zip(names, refs):
        _check(name, got[name], ref, CHUNK_BLOCKS[name], 2e-2, errs)
    say("[gla maxsize] rel-L2: " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))


def test_sscan_past_int32_elements(coracle):
    """Selective scan with N=16 entries per channel at B=2, T=2^20+37,
    D=1024 (x, delta, y, dx, ddelta past 2^31 elements; time split into
    segments), h0 and dh_T given: y, h_T, dx, ddelta and dh0 on 7 sampled
    channels of both batch rows, dA on those channels (summed over the
    batch); dB and dC (sums over every channel) finite."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, rel_l2, say, to_dev
    B, T, D, N = 2, (1 << 20) + 37, 1024, 16
    assert B * T * D > 2 ** 31
    sel = np.array([0, 1, 63, 64, 511, 1022, 1023], dtype=np.int64)
    say(f"[sscan maxsize] B={B} T={T} D={D} N={N} channels={sel.tolist()}")
    d = dev()
    g = torch.Generator(device=d)
    g.manual_seed(2034)
    ci = syn.sscan_inputs(B, T, len(sel), N, 2034, h0_scale=0.1, dhT_scale=0.1)
    lo, hi = math.log(1e-3), math.log(1e-1)
    x = torch.randn(B, T, D, device=d, generator=g)
    dl = torch.empty(B, T, D, device=d).uniform_(lo, hi, generator=g).exp_()
    dy = torch.randn(B, T, D, device=d, generator=g)
    h0 = torch.randn(B, D, N, device=d, generator=g) * 0.1
    dhT = torch.randn(B, D, N, device=d, generator=g) * 0.1
    # A is the same s4d row for every channel; B and C are shared by all
    # channels, so they come whole from the generator
    A = torch.from_numpy(np.tile(ci.A[:1], (D, 1))).to(d)
    Bm, Cm = to_dev(ci.Bm), to_dev(ci.Cm)
    idx = torch.from_numpy(sel).to(d)
    for t, val in ((x, ci.x), (dl, ci.delta), (dy, ci.dy)):
        t.index_copy_(2, idx, to_dev(val))
    for t, val in ((h0, ci.h0), (dhT, ci.dhT)):
        t.index_copy_(1, idx, to_dev(val))
    assert torch.equal(A.index_select(0, idx), to_dev(ci.A))
    y, hT, ck = cla.selective_scan(x, dl, A, Bm, Cm, h0, save_ckpt=True)
    gr = cla.selective_scan_bwd(x, dl, A, Bm, Cm, h0, dy, dhT, ckpt=ck)
    torch.cuda.synchronize()
    names = ("y", "hT", "dx", "ddelta", "dA", "dB", "dC", "dh0")
    out = (y, hT) + tuple(gr)
    for name, t in zip(names, out):
        assert bool(torch.isfinite(t).all()), name
    got = {"y": y.index_select(2, idx), "dx": gr[0].index_select(2, idx),
           "ddelta": gr[1].index_select(2, idx), "hT": hT.index_select(1, idx),
           "dh0": gr[5].index_select(1, idx), "dA": gr[2].index_select(0, idx)}
    got = {k_: v_.cpu().numpy().astype(np.float64) for k_, v_ in got.items()}
    ns = len(sel)
    # the oracle's units are (batch, channel) pairs, batch-major
    for k_ in ("y", "dx", "ddelta"):
        got[k_] = got[k_].transpose(0, 2, 1).reshape(B * ns, T)
    for k_ in ("hT", "dh0"):
        got[k_] = got[k_].reshape(B * ns, N)
    del x, dl, dy, y, gr, out, ck
    torch.cuda.empty_cache()
    say("[sscan maxsize] oracle on the sampled channels")
    yr, hTr = coracle.sscan_fwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0)
    dxr, ddr, dAr, _, _, dh0r = coracle.sscan_bwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0,
                                                 ci.dy, ci.dhT)
    dAr = dAr.reshape(B, ns, N).sum(axis=0)
    errs = {}
    for name, ref, blk in (("y", yr, (1, 1024)), ("dx", dxr, (1, 1024)),
                           ("ddelta", ddr, (1, 1024)), ("hT", hTr, (1,)),
                           ("dh0", dh0r, (1,))):
        _check(name, got[name], ref, blk, 1e-5, errs)
    # dA[d] sums its terms over all B*T steps in fp32 accumulators; the 1e-5
    # bar holds for sums of up to 32768 steps (the full-size workloads), and
    # the accumulated rounding grows like the square root of the count, so
    # each channel's 16 entries get that bar scaled to B*T steps (8.0e-5 here);
    # the sampled channels together keep the plain bar
    errs["dA"] = rel_l2(got["dA"], dAr)
    assert errs["dA"] <= 1e-5, ("dA", errs["dA"])
    tol_a = 1e-5 * math.sqrt(B * T / 32768)
    _check("dA_ch", got["dA"], dAr, (1,), tol_a, errs)
    say("[sscan maxsize] rel-L2: " + ", ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()))
