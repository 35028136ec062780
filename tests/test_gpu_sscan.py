"""Selective scan with N state entries per channel (Mamba-1's recurrence)
against the float64 oracle, through the C ABI (GPU).

The oracle runs on the exact device inputs (fp32).  The bar is the fp32
scan's: relative L2 error <= 1e-5 per output tensor.  Cases cover one step,
ragged T (not a multiple of the 32-step tile), D not a multiple of the
64-channel workgroup, N in {4, 8, 16}, strong and weak decays, no decay
(A = 0), initial state and final-state gradient present or absent, T = 0,
stitched pieces, the backward with and without the forward's checkpoints,
bit-identical repeats, and the full-size workload on sampled channels.  Every
case with few (sequence, 64-channel group) units and T > 96 runs with time
split into segments (up to 94 here); the large cases run unsplit.
"""

import numpy as np
import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("y", "hT", "dx", "ddelta", "dA", "dB", "dC", "dh0")


def _dev(ci):
    from gpu_util import to_dev
    return [to_dev(v) for v in (ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, ci.dy, ci.dhT)]


def _run(ci, use_ckpt=True):
    import torch
    import chunkwise_linear_attention_amd as cla
    x, dl, A, Bm, Cm, h0, dy, dhT = _dev(ci)
    y, hT, ck = cla.selective_scan(x, dl, A, Bm, Cm, h0, save_ckpt=True)
    g = cla.selective_scan_bwd(x, dl, A, Bm, Cm, h0, dy, dhT, ckpt=ck if use_ckpt else None)
    torch.cuda.synchronize()
    return (y, hT) + tuple(g)


def _oracle_all(coracle, ci):
    Bt, T, D = ci.x.shape
    N = ci.A.shape[1]
    y, hT = coracle.sscan_fwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0)
    dx, dd, dA, dB, dC, dh0 = coracle.sscan_bwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0,
                                                ci.dy, ci.dhT)
    # per-unit [b*D + d, T] -> [B, T, D]
    tr = lambda u: u.reshape(Bt, D, T).transpose(0, 2, 1)
    return (tr(y), hT.reshape(Bt, D, N), tr(dx), tr(dd), dA.reshape(Bt, D, N).sum(axis=0),
            dB, dC, dh0.reshape(Bt, D, N))


def _compare(got, ref):
    from gpu_util import rel_l2, to_np
    errs = {}
    for name, g, r in zip(NAMES, got, ref):
        errs[name] = rel_l2(to_np(g), r)
    return errs


CASES = [
    # (B, T, D, N, delta, A, h0, dhT, seed)
    (1, 1, 64, 16, ("loguniform", 1e-3, 1e-1), "s4d", False, False, 1),
    (2, 33, 64, 16, ("loguniform", 1e-3, 1e-1), "s4d", True, True, 2),
    (1, 100, 100, 16, ("loguniform", 1e-3, 1e-1), ("uniform", -4.0, -0.1), True, False, 3),
    (3, 257, 132, 8, ("loguniform", 1e-3, 1e-1), ("uniform", -2.0, -0.5), False, True, 4),
    (2, 64, 192, 4, ("loguniform", 1e-2, 1.0), "s4d", True, True, 5),
    (1, 1000, 256, 16, ("loguniform", 1e-2, 1.0), "s4d", True, True, 6),
    (2, 500, 68, 16, ("loguniform", 1e-3, 1e-1), ("uniform", -8.0, -0.1), True, True, 7),
    (1, 300, 64, 16, ("loguniform", 1e-4, 1e-2), ("const", 0.0), True, True, 8),   # no decay
    (1, 77, 64, 16, ("loguniform", 0.5, 5.0), "s4d", True, True, 9),               # strong decays
    (4, 2048, 320, 16, ("loguniform", 1e-3, 1e-1), "s4d", False, False, 10),
    # few (sequence, channel group) units: time split into segments of whole
    # 32-step tiles (every case above with T > 96 is split as well)
    (1, 3000, 64, 16, ("loguniform", 1e-3, 1e-1), ("uniform", -2.0, -0.1), True, True, 11),
    (2, 1000, 64, 8, ("loguniform", 1e-2, 1.0), "s4d", True, True, 12),
    # enough units: no split
    (8, 200, 4096, 4, ("loguniform", 1e-3, 1e-1), "s4d", True, True, 13),
]


@pytest.mark.parametrize("B,T,D,N,delta,A,h0,dhT,seed", CASES)
def test_sscan_parity(coracle, B, T, D, N, delta, A, h0, dhT, seed):
    from gpu_util import say
    ci = syn.sscan_inputs(B, T, D, N, seed, delta=delta, A=A, h0_scale=0.5 if h0 else None,
                          dhT_scale=0.5 if dhT else None)
    say(f"[sscan] B={B} T={T} D={D} N={N} delta={delta} A={A} h0={h0} dhT={dhT} seed={seed}")
    errs = _compare(_run(ci), _oracle_all(coracle, ci))
    say("[sscan] rel-L2 " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL}
    assert not bad, errs


def test_sscan_checkpoints_optional_and_deterministic():
    """The backward without the forward's checkpoints (it recomputes them) gives
    bit-identical results, and repeated calls are bit-identical."""
    import torch
    from gpu_util import say
    say("[sscan] checkpoints given / recomputed, repeats")
    ci = syn.sscan_inputs(2, 300, 128, 16, 21, h0_scale=0.3, dhT_scale=0.3)
    a = _run(ci, use_ckpt=True)
    b = _run(ci, use_ckpt=False)
    c = _run(ci, use_ckpt=True)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_sscan_empty_and_stitched(coracle):
    """T = 0 returns h0 as the final state and dhT as dh0; two pieces run
    back to back (the second from the first's final state) match one run,
    forward and backward (the first piece's dhT is the second's dh0)."""
    import torch
    import chunkwise_linear_attention_amd as cla
    from gpu_util import rel_l2, say, to_dev, to_np
    say("[sscan] T = 0 and stitched pieces")
    ci = syn.sscan_inputs(2, 0, 64, 16, 22, h0_scale=0.5, dhT_scale=0.5)
    x, dl, A, Bm, Cm, h0, dy, dhT = _dev(ci)
    y, hT = cla.selective_scan(x, dl, A, Bm, Cm, h0)
    g = cla.selective_scan_bwd(x, dl, A, Bm, Cm, h0, dy, dhT)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(hT, h0) and torch.equal(g[5], dhT)
    assert torch.count_nonzero(g[2]) == 0
    ci = syn.sscan_inputs(2, 150, 128, 16, 23, h0_scale=0.5, dhT_scale=0.5)
    x, dl, A, Bm, Cm, h0, dy, dhT = _dev(ci)
    T1 = 61
    piece = lambda t, lo, hi: t[:, lo:hi].contiguous()
    ya, ha = cla.selective_scan(piece(x, 0, T1), piece(dl, 0, T1), A, piece(Bm, 0, T1),
                                piece(Cm, 0, T1), h0)
    yb, hb = cla.selective_scan(piece(x, T1, 150), piece(dl, T1, 150), A, piece(Bm, T1, 150),
                                piece(Cm, T1, 150), ha)
    gb = cla.selective_scan_bwd(piece(x, T1, 150), piece(dl, T1, 150), A, piece(Bm, T1, 150),
                                piece(Cm, T1, 150), ha, piece(dy, T1, 150), dhT)
    ga = cla.selective_scan_bwd(piece(x, 0, T1), piece(dl, 0, T1), A, piece(Bm, 0, T1),
                                piece(Cm, 0, T1), h0, piece(dy, 0, T1), gb[5])
    torch.cuda.synchronize()
    ref = _oracle_all(coracle, ci)
    got = (torch.cat([ya, yb], 1), hb, torch.cat([ga[0], gb[0]], 1), torch.cat([ga[1], gb[1]], 1),
           ga[2] + gb[2], torch.cat([ga[3], gb[3]], 1), torch.cat([ga[4], gb[4]], 1), ga[5])
    errs = _compare(got, ref)
    say("[sscan] stitched rel-L2 " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs


@pytest.mark.parametrize("wl", ["sscan_mamba", "sscan_b1"])
def test_sscan_workload_sampled(coracle, wl):
    """The bench workloads (B=8, T=4096, D=5120, N=16; B=1, T=32768, D=2048,
    N=16 with time split into 16 segments) at full size, in the launch
    configuration the bench times: y, h_T, dx, ddelta and dh0 on sampled
    channels, dA on sampled channels summed over the batch, dB and dC for one
    whole sequence; every output finite.  The bar holds for the whole sampled
    tensors and for every 1024-step block of each sampled channel."""
    import torch
    from gpu_util import block_rel_l2, rel_l2, say, to_np
    ci = syn.WORKLOADS[wl].make()
    Bt, T, D = ci.x.shape
    N = ci.A.shape[1]
    say(f"[sscan workload] {wl} shape B={Bt} T={T} D={D} N={N}")
    out = _run(ci)
    for name, t in zip(NAMES, out):
        if t is not None:
            assert bool(torch.isfinite(t).all()), name
    ds = np.array(sorted({0, 1, D // 7, D // 2, D - 2, D - 1}))
    bs = sorted({0, Bt // 2, Bt - 1})
    chans = np.array([b * D + d for b in bs for d in ds], dtype=np.int64)
    y, hT = coracle.sscan_fwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, chans=chans)
    dx, dd, _, _, _, dh0 = coracle.sscan_bwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, ci.dy,
                                             ci.dhT, chans=chans)
    gy, ghT, gdx, gdd = (to_np(t) for t in out[:2] + out[2:4])
    errs = {}
    bsel, dsel = chans // D, chans % D
    # whole sampled tensors, and every 1024-step block of each sampled channel
    for nm, g, r in (("y", gy[bsel, :, dsel], y), ("dx", gdx[bsel, :, dsel], dx),
                     ("ddelta", gdd[bsel, :, dsel], dd)):
        errs[nm] = rel_l2(g, r)
        errs[nm + "_blk"] = block_rel_l2(g, r, (1, 1024))[0]
    errs["hT"] = rel_l2(ghT[bsel, dsel], hT)
    errs["hT_blk"] = block_rel_l2(ghT[bsel, dsel], hT, (1,))[0]
    if out[7] is not None:
        errs["dh0"] = rel_l2(to_np(out[7])[bsel, dsel], dh0)
    # dA on sampled channels: all sequences
    chA = np.array([b * D + d for d in ds for b in range(Bt)], dtype=np.int64)
    rA = coracle.sscan_bwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, ci.dy, ci.dhT,
                           chans=chA)[2].reshape(len(ds), Bt, N).sum(axis=1)
    errs["dA"] = rel_l2(to_np(out[4])[ds], rA)
    # dB, dC of one sequence: every channel
    sb = min(5, Bt - 1)
    b5 = np.arange(sb * D, (sb + 1) * D, dtype=np.int64)
    rB, rC = coracle.sscan_bwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, ci.dy, ci.dhT,
                               chans=b5)[3:5]
    errs["dB"] = rel_l2(to_np(out[5])[sb], rB[sb])
    errs["dC"] = rel_l2(to_np(out[6])[sb], rC[sb])
    errs["dB_blk"] = block_rel_l2(to_np(out[5])[sb], rB[sb], (1024,))[0]
    errs["dC_blk"] = block_rel_l2(to_np(out[6])[sb], rC[sb], (1024,))[0]
    say(f"[sscan workload] {wl} rel-L2 " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL for v in errs.values()), errs
