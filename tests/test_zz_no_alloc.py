"""The diagonal-scan forward that allocates nothing (cla_scan_fwd_noalloc),
called through the C ABI on the GPU and compared with cla_scan_fwd, the entry
point that takes a caller workspace, and with the float64 oracle.

Both entry points run the same kernels on the same plan, so their outputs
must be bit-identical; against the oracle the fp32 bar applies (relative L2
error <= 1e-5).  The shapes split the time axis into segments, so the fixed
device array holds the segment pairs: the largest such need (B=1, T=65536,
D=64: 511 segments of 64 channels), the small scan workload (B=1, T=4096,
D=64) and a smaller ragged one (D not a multiple of 4).  Calls follow each
other with no synchronisation in between, the later ones smaller, so stale
pairs left in the array by an earlier call would show.
"""

import ctypes

import numpy as np
import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _dev_inputs(inp):
    from gpu_util import to_dev
    return to_dev(inp.a), to_dev(inp.b), to_dev(inp.h0)


def _fwd_workspace(L, a, b, h0, stream):
    import torch
    B, T, D = a.shape
    h = torch.empty_like(a)
    hT = torch.empty((B, D), dtype=torch.float32, device=a.device)
    nbytes = int(L.cla_scan_workspace_bytes(B, T, D))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=a.device)
    st = L.cla_scan_fwd(a.data_ptr(), b.data_ptr(), h0.data_ptr() if h0 is not None else None,
                        h.data_ptr(), hT.data_ptr(), B, T, D, ws.data_ptr(), nbytes, stream)
    assert st == 0, L.cla_status_string(st)
    return h, hT, ws


def _fwd_noalloc(L, a, b, h0, stream):
    import torch
    B, T, D = a.shape
    h = torch.empty_like(a)
    hT = torch.empty((B, D), dtype=torch.float32, device=a.device)
    st = L.cla_scan_fwd_noalloc(a.data_ptr(), b.data_ptr(),
                                h0.data_ptr() if h0 is not None else None,
                                h.data_ptr(), hT.data_ptr(), B, T, D, stream)
    assert st == 0, L.cla_status_string(st)
    return h, hT


# (B, T, D, h0, seed), largest first
SEQUENCE = [
    (1, 65536, 64, True, 31),
    (1, 4096, 64, False, 1001),
    (1, 1000, 20, True, 32),
]


def test_noalloc_matches_workspace_entry_point(coracle):
    import torch
    from chunkwise_linear_attention_amd import _lib
    from gpu_util import dev, rel_l2, say, to_np
    L = _lib.lib()
    stream = torch.cuda.current_stream(dev()).cuda_stream
    for B, T, D, _, _ in SEQUENCE:
        assert 0 < L.cla_scan_workspace_bytes(B, T, D) <= ctypes.c_size_t(262144).value
    inps = [syn.scan_inputs(B, T, D, seed, h0=h0) for B, T, D, h0, seed in SEQUENCE]
    devs = [_dev_inputs(i) for i in inps]
    # two rounds of calls, each round largest first, nothing synchronised
    # between the calls of a round
    for rnd in range(2):
        outs = []
        for (B, T, D, _, _), (a, b, h0) in zip(SEQUENCE, devs):
            say(f"[no_alloc] round {rnd}: cla_scan_fwd_noalloc B={B} T={T} D={D}")
            na = _fwd_noalloc(L, a, b, h0, stream)
            ref = _fwd_workspace(L, a, b, h0, stream)
            outs.append((na, ref))
        torch.cuda.synchronize()
        for (B, T, D, _, _), inp, ((h, hT), (hw, hTw, _)) in zip(SEQUENCE, inps, outs):
            assert torch.equal(h, hw) and torch.equal(hT, hTw), (B, T, D)
            hr, hTr = coracle.scan_fwd(inp.a, inp.b, inp.h0)
            eh, ehT = rel_l2(to_np(h), hr), rel_l2(to_np(hT), hTr)
            say(f"[no_alloc] round {rnd} B={B} T={T} D={D}: rel_l2 h {eh:.2e} hT {ehT:.2e}")
            assert eh <= TOL and ehT <= TOL, (B, T, D, eh, ehT)


def test_noalloc_without_segments_and_empty():
    """A shape that fills the GPU without a time split uses no array; T = 0
    copies h0 to hT."""
    import torch
    from chunkwise_linear_attention_amd import _lib
    from gpu_util import dev, say
    L = _lib.lib()
    stream = torch.cuda.current_stream(dev()).cuda_stream
    say("[no_alloc] B=8 T=256 D=4096 (no time split)")
    inp = syn.scan_inputs(8, 256, 4096, 33, h0=True)
    a, b, h0 = _dev_inputs(inp)
    assert L.cla_scan_workspace_bytes(8, 256, 4096) == 0
    h, hT = _fwd_noalloc(L, a, b, h0, stream)
    hw, hTw, _ = _fwd_workspace(L, a, b, h0, stream)
    torch.cuda.synchronize()
    assert torch.equal(h, hw) and torch.equal(hT, hTw)
    say("[no_alloc] T=0")
    e = torch.empty((2, 0, 5), dtype=torch.float32, device=dev())
    h0 = torch.arange(10, dtype=torch.float32, device=dev()).reshape(2, 5)
    hT = torch.full((2, 5), -1.0, device=dev())
    st = L.cla_scan_fwd_noalloc(e.data_ptr(), e.data_ptr(), h0.data_ptr(), e.data_ptr(),
                                hT.data_ptr(), 2, 0, 5, stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(hT, h0)
