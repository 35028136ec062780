"""The torch.autograd wrappers (GPU): loss.backward() through each Function
gives exactly the gradients of the direct backward calls (the wrappers only
forward the calls), including outputs left out of the loss."""

import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu


def _dev(x, grad=True):
    from gpu_util import to_dev
    t = to_dev(x)
    return None if t is None else t.requires_grad_(grad)


def test_scan_fn():
    import torch
    import chunkwise_linear_attention_amd as cla
    from chunkwise_linear_attention_amd.autograd import scan_fn
    from gpu_util import say
    say("[autograd] scan")
    si = syn.scan_inputs(2, 300, 68, 41, h0=True, dhT=True)
    a, b, h0 = _dev(si.a), _dev(si.b), _dev(si.h0)
    dh, dhT = _dev(si.dh, False), _dev(si.dhT, False)
    h, hT = scan_fn(a, b, h0)
    ((h * dh).sum() + (hT * dhT).sum()).backward()
    h2, _ = cla.scan(a.detach(), b.detach(), h0.detach())
    da, db, dh0 = cla.scan_bwd(a.detach(), h2, h0.detach(), dh, dhT)
    assert torch.equal(a.grad, da) and torch.equal(b.grad, db) and torch.equal(h0.grad, dh0)


def test_chunked_linear_attn_fn():
    import torch
    import chunkwise_linear_attention_amd as cla
    from chunkwise_linear_attention_amd.autograd import chunked_linear_attn_fn
    from gpu_util import say
    say("[autograd] chunked linear attention (o only in the loss)")
    ci = syn.chunk_inputs(1, 2, 300, 64, 64, 42, qk_scale=0.125, S0_scale=0.1)
    q, k, v, l, S0 = (_dev(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0))
    dO = _dev(ci.dO, False)
    o, ST = chunked_linear_attn_fn(q, k, v, l, S0)
    (o.float() * dO.float()).sum().backward()
    qd, kd, vd, ld, S0d = (t.detach() for t in (q, k, v, l, S0))
    _, _, saved = cla.chunked_linear_attn(qd, kd, vd, ld, S0d, save_states=True)
    ref = cla.chunked_linear_attn_bwd(qd, kd, vd, ld, S0d, dO, None, saved=saved)
    for g, r in zip((q.grad, k.grad, v.grad, l.grad, S0.grad), ref):
        assert torch.equal(g, r)


def test_gla_fn():
    import torch
    import chunkwise_linear_attention_amd as cla
    from chunkwise_linear_attention_amd.autograd import gla_fn
    from gpu_util import say
    say("[autograd] gated linear attention")
    gi = syn.gla_inputs(1, 2, 200, 64, 64, 43, S0_scale=0.1, dST_scale=0.1)
    q, k, v, l, S0 = (_dev(x) for x in (gi.q, gi.k, gi.v, gi.l, gi.S0))
    dO, dST = _dev(gi.dO, False), _dev(gi.dST, False)
    o, ST = gla_fn(q, k, v, l, S0)
    ((o.float() * dO.float()).sum() + (ST * dST).sum()).backward()
    ref = cla.gla_bwd(q.detach(), k.detach(), v.detach(), l.detach(), S0.detach(), dO, dST)
    for g, r in zip((q.grad, k.grad, v.grad, l.grad, S0.grad), ref):
        assert torch.equal(g, r)


def test_selective_scan_fn():
    import torch
    import chunkwise_linear_attention_amd as cla
    from chunkwise_linear_attention_amd.autograd import selective_scan_fn
    from gpu_util import say
    say("[autograd] selective scan (h_T only in the loss, then y only)")
    si = syn.sscan_inputs(2, 500, 128, 16, 44, h0_scale=0.5, dhT_scale=0.5)
    for use_y in (False, True):
        x, dl, A, Bm, Cm, h0 = (_dev(t) for t in (si.x, si.delta, si.A, si.Bm, si.Cm, si.h0))
        dy, dhT = _dev(si.dy, False), _dev(si.dhT, False)
        y, hT = selective_scan_fn(x, dl, A, Bm, Cm, h0)
        loss = (y * dy).sum() if use_y else (hT * dhT).sum()
        loss.backward()
        args = tuple(t.detach() for t in (x, dl, A, Bm, Cm, h0))
        _, _, ck = cla.selective_scan(*args, save_ckpt=True)
        ref = cla.selective_scan_bwd(*args, dy if use_y else torch.zeros_like(dy),
                                     None if use_y else dhT, ckpt=ck)
        for g, r in zip((x.grad, dl.grad, A.grad, Bm.grad, Cm.grad, h0.grad), ref):
            assert torch.equal(g, r)
