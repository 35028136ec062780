"""Parity of the HIP diagonal scan (forward and backward) against the float64
oracle, through the C ABI (GPU).

Tolerance: relative L2 error <= 1e-5 per output tensor (fp32 path), computed
in float64 against the oracle run on the exact device inputs.
"""

import numpy as np
import pytest

import synthetic as syn
from oracle import scan as osc

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _run(inp, want_final=True):
    import chunkwise_linear_attention_amd as cla
    from gpu_util import to_dev
    a, b, dh = to_dev(inp.a), to_dev(inp.b), to_dev(inp.dh)
    h0, dhT = to_dev(inp.h0), to_dev(inp.dhT)
    h, hT = cla.scan(a, b, h0, want_final=want_final)
    da, db, dh0 = cla.scan_bwd(a, h, h0, dh, dhT)
    return h, hT, da, db, dh0


# blocks of the error measure: each batch row, 1024 steps, 64 channels (one
# workgroup's channel group); final states per batch row and channel group
SEQ_BLOCKS = (1, 1024, 64)
ROW_BLOCKS = (1, 64)


def _check(inp, got, coracle):
    """Whole tensors and every block within the bar."""
    from gpu_util import block_rel_l2, rel_l2, to_np
    h, hT, da, db, dh0 = got
    hr, hTr = coracle.scan_fwd(inp.a, inp.b, inp.h0)
    # the backward oracle's h input is the oracle's own forward output, stored
    # in fp32 as the library stores h (never the device's h)
    dar, dbr, dh0r = coracle.scan_bwd(inp.a, hr.astype(np.float32), inp.h0, inp.dh, inp.dhT)
    pairs = {"h": (to_np(h), hr, SEQ_BLOCKS), "da": (to_np(da), dar, SEQ_BLOCKS),
             "db": (to_np(db), dbr, SEQ_BLOCKS), "dh0": (to_np(dh0), dh0r, ROW_BLOCKS)}
    if hT is not None:
        pairs["hT"] = (to_np(hT), hTr, ROW_BLOCKS)
    errs = {}
    for k, (x, r, blk) in pairs.items():
        errs[k] = rel_l2(x, r)
        errs[k + "_blk"] = block_rel_l2(x, r, blk)[0]
    for k, e in errs.items():
        assert e <= TOL, (k, e, errs)
    return errs


CASES = [
    # (B, T, D, h0, dhT, seed): ragged time tails, D not a multiple of 4,
    # single channel / single step, several segments and the sweep path
    (1, 1, 1, False, False, 1),
    (1, 2, 3, True, True, 2),
    (2, 5, 3, True, False, 3),
    (1, 127, 64, False, True, 4),
    (1, 129, 64, True, True, 5),
    (3, 1000, 67, True, True, 6),
    (2, 777, 128, False, False, 7),
    (1, 4096, 64, False, False, 8),
    (4, 3000, 1024, True, True, 9),
    (1, 300, 32768, True, True, 10),      # 512 channel groups: no time split
    (2, 513, 16384 + 4, True, False, 11),
]


@pytest.mark.parametrize("B,T,D,h0,dhT,seed", CASES)
def test_scan_parity(coracle, B, T, D, h0, dhT, seed):
    from gpu_util import say
    say(f"[scan parity] B={B} T={T} D={D} h0={h0} dhT={dhT} seed={seed}")
    inp = syn.scan_inputs(B, T, D, seed, delta=(1e-3, 0.5), h0=h0, dhT=dhT)
    _check(inp, _run(inp), coracle)


@pytest.mark.parametrize("const", [0.0, 1.0])
def test_scan_special_decays(coracle, const):
    from gpu_util import say, to_np
    say(f"[scan special] a = {const}")
    inp = syn.scan_inputs(2, 300, 20, 21, h0=True, dhT=True, a_const=const)
    got = _run(inp)
    _check(inp, got, coracle)
    h = to_np(got[0])
    if const == 0.0:
        np.testing.assert_array_equal(h, inp.b.astype(np.float64))
    else:
        ref = np.cumsum(inp.b.astype(np.float64), axis=1) + inp.h0[:, None, :]
        assert np.max(np.abs(h - ref)) < 1e-3


@pytest.mark.parametrize("h0", ["null", "zeros"])
def test_scan_small_workload_full(coracle, h0):
    """The small workload (B=1, T=4096, D=64: one channel group, time split
    into 32 segments) with h0 given as NULL and as explicit zeros; both give
    the same results, bit for bit."""
    import torch
    from gpu_util import say
    say(f"[scan workload] B=1 T=4096 D=64 (seed 1001) h0={h0}")
    inp = syn.WORKLOADS["scan_small"].make()
    if h0 == "zeros":
        inp.h0 = np.zeros((1, 64), dtype=np.float32)
    got = _run(inp)
    errs = _check(inp, got, coracle)
    say("[scan workload] rel-L2 " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    if h0 == "zeros":
        inp.h0 = None
        ref = _run(inp)
        for x, y in zip(got, ref):
            assert torch.equal(x, y)


def test_scan_empty_sequence():
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import dev, say
    say("[scan empty] T=0")
    a = torch.zeros((2, 0, 5), device=dev())
    h0 = torch.randn((2, 5), device=dev())
    h, hT = cla.scan(a, a.clone(), h0)
    assert h.shape == (2, 0, 5)
    assert torch.equal(hT, h0)
    dhT = torch.randn((2, 5), device=dev())
    da, db, dh0 = cla.scan_bwd(a, a.clone(), h0, a.clone(), dhT)
    assert torch.equal(dh0, dhT)
    _, hT0 = cla.scan(a, a.clone(), None)
    assert torch.count_nonzero(hT0) == 0


def test_scan_stitched_pieces(coracle):
    """Two pieces: the second starts from the first's final state; the first's
    backward receives the second's dh0 as its final-state gradient."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import rel_l2, say, to_dev, to_np
    say("[scan stitched] B=2 T=700+333 D=96")
    inp = syn.scan_inputs(2, 1033, 96, 31, h0=True, dhT=True)
    a, b, dh = to_dev(inp.a), to_dev(inp.b), to_dev(inp.dh)
    h0, dhT = to_dev(inp.h0), to_dev(inp.dhT)
    s = 700
    a1, a2 = a[:, :s].contiguous(), a[:, s:].contiguous()
    b1, b2 = b[:, :s].contiguous(), b[:, s:].contiguous()
    h1, hT1 = cla.scan(a1, b1, h0)
    h2, hT2 = cla.scan(a2, b2, hT1)
    da2, db2, dmid = cla.scan_bwd(a2, h2, hT1, dh[:, s:].contiguous(), dhT)
    da1, db1, dh0 = cla.scan_bwd(a1, h1, h0, dh[:, :s].contiguous(), dmid)
    hr, hTr = osc.scan_loop(inp.a, inp.b, inp.h0)
    hcat = torch.cat([h1, h2], 1)
    dar, dbr, dh0r = osc.scan_bwd_loop(inp.a, hr, inp.h0, inp.dh, inp.dhT)
    assert rel_l2(to_np(hcat), hr) <= TOL
    assert rel_l2(to_np(hT2), hTr) <= TOL
    assert rel_l2(to_np(torch.cat([da1, da2], 1)), dar) <= TOL
    assert rel_l2(to_np(torch.cat([db1, db2], 1)), dbr) <= TOL
    assert rel_l2(to_np(dh0), dh0r) <= TOL


def test_scan_deterministic():
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import say, to_dev
    say("[scan determinism] B=1 T=4096 D=64 and B=4 T=3000 D=1024")
    for B, T, D in ((1, 4096, 64), (4, 3000, 1024)):
        inp = syn.scan_inputs(B, T, D, 41, h0=True, dhT=True)
        a, b, dh = to_dev(inp.a), to_dev(inp.b), to_dev(inp.dh)
        h0, dhT = to_dev(inp.h0), to_dev(inp.dhT)
        r1 = [cla.scan(a, b, h0), cla.scan_bwd(a, cla.scan(a, b, h0)[0], h0, dh, dhT)]
        r2 = [cla.scan(a, b, h0), cla.scan_bwd(a, cla.scan(a, b, h0)[0], h0, dh, dhT)]
        for x, y in zip([t for g in r1 for t in g], [t for g in r2 for t in g]):
            assert torch.equal(x, y)


def test_scan_large_workload_full(coracle):
    """The B=8, T=16384, D=4096 workload in the bench's launch configuration
    (XCD-ordered workgroups), compared with the oracle on every channel, in
    slabs of 512 channels: the whole slab and every block (batch row, 1024
    steps, 64 channels) within the bar."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import block_rel_l2, rel_l2, say, to_dev
    say("[scan large] B=8 T=16384 D=4096 (seed 1002), every channel")
    inp = syn.WORKLOADS["scan_large"].make()
    a, b, dh = to_dev(inp.a), to_dev(inp.b), to_dev(inp.dh)
    h0 = to_dev(inp.h0)
    h, hT = cla.scan(a, b, h0)
    da, db, dh0 = cla.scan_bwd(a, h, h0, dh, None)
    torch.cuda.synchronize()
    del a, b, dh
    h_full = h.cpu().numpy()
    worst = {}
    for d0 in range(0, 4096, 512):
        sl = slice(d0, d0 + 512)
        hr, hTr = coracle.scan_fwd(inp.a, inp.b, inp.h0, drange=(d0, d0 + 512))
        # the backward oracle runs on the slab with the oracle's own h (fp32)
        dar, dbr, dh0r = coracle.scan_bwd(inp.a[:, :, sl], hr.astype(np.float32),
                                          None if inp.h0 is None else inp.h0[:, sl],
                                          inp.dh[:, :, sl], None)
        pairs = {"h": (h_full[:, :, sl], hr, SEQ_BLOCKS),
                 "hT": (hT[:, sl].cpu().numpy(), hTr, ROW_BLOCKS),
                 "da": (da[:, :, sl].cpu().numpy(), dar, SEQ_BLOCKS),
                 "db": (db[:, :, sl].cpu().numpy(), dbr, SEQ_BLOCKS),
                 "dh0": (dh0[:, sl].cpu().numpy(), dh0r, ROW_BLOCKS)}
        for k, (x, r, blk) in pairs.items():
            e = rel_l2(x, r)
            eb, at = block_rel_l2(x, r, blk)
            assert e <= TOL, (k, d0, e)
            assert eb <= TOL, (k, d0, at, eb)
            worst[k] = max(worst.get(k, 0.0), e)
            worst[k + "_blk"] = max(worst.get(k + "_blk", 0.0), eb)
        del hr, dar, dbr
    say("[scan large] worst rel-L2 over slabs " +
        ", ".join(f"{k}={v:.2e}" for k, v in worst.items()))
