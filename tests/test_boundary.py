"""The C ABI boundary on the host (CPU only, no GPU calls).

The library must load, export every function include/cla.h declares, and
reject bad arguments with the documented status codes before any launch.
Fake non-NULL addresses are used for pointers the checks only compare; every
call here is meant to return before the library touches the device.

So that a regression in that validation can never hand a fake address to a
real GPU, the checks run in a child process started with every GPU hidden
(HIP_VISIBLE_DEVICES, ROCR_VISIBLE_DEVICES and CUDA_VISIBLE_DEVICES set
empty), which confirms that it sees no device before it loads the library.
"""

import ctypes
import os
import subprocess
import sys

import pytest

from chunkwise_linear_attention_amd import _lib

OK, NULL, SHAPE, UNSUP, WS, ALIAS = 0, 1, 2, 3, 4, 5

# distinct fake device addresses, far apart so that ranges never overlap
A, B_, C, D_, E, F, G, H_, I, J, K, L = (0x10_0000_0000 * (i + 1) for i in range(12))

_CHILD_FLAG = "CLA_BOUNDARY_GPU_HIDDEN"
IN_CHILD = os.environ.get(_CHILD_FLAG) == "1"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_checks_in_gpu_free_child():
    """Run every check below in a child process that sees no GPU."""
    if IN_CHILD:
        pytest.skip("this is the child")
    env = dict(os.environ)
    env.update({_CHILD_FLAG: "1", "HIP_VISIBLE_DEVICES": "", "ROCR_VISIBLE_DEVICES": "",
                "CUDA_VISIBLE_DEVICES": ""})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.abspath(__file__)], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert " passed" in r.stdout and "failed" not in r.stdout


@pytest.fixture(scope="module")
def lib():
    if not IN_CHILD:
        pytest.skip("runs in the GPU-free child process")
    import torch
    # counting devices does not initialise the GPU; with every device hidden
    # the count must be 0 before any fake address reaches the library
    n = torch.cuda.device_count()
    if n != 0:
        pytest.fail(f"{n} GPU(s) visible in the child; refusing to pass fake addresses")
    # a differently built copy of the library (the host-sanitizer run)
    other = os.environ.get("CLA_BOUNDARY_LIB")
    if other:
        _lib.LIB_PATH = other
    return _lib.lib()


def test_exports_every_declared_symbol(lib):
    names = _lib.header_symbols()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.cla_status_string(code).decode().startswith(name)
    assert b"UNKNOWN" in lib.cla_status_string(99)
    assert lib.cla_version().startswith(b"cla")


def test_scan_workspace_sizes(lib):
    # a batch-and-channel count that fills the GPU needs no workspace
    assert lib.cla_scan_workspace_bytes(8, 16384, 4096) == 0
    # one 64-channel group is split into 32 segments of 128 steps
    assert lib.cla_scan_workspace_bytes(1, 4096, 64) == 31 * 64 * 8
    assert lib.cla_scan_workspace_bytes(-1, 4, 4) == 0
    assert lib.cla_scan_workspace_bytes(1, 0, 4) == 0


def test_scan_fwd_validation(lib):
    f = lib.cla_scan_fwd
    assert f(A, B_, None, C, None, -1, 4, 4, None, 0, None) == SHAPE
    assert f(A, B_, None, C, None, 1, -4, 4, None, 0, None) == SHAPE
    assert f(None, B_, None, C, None, 1, 4, 4, None, 0, None) == NULL
    assert f(A, None, None, C, None, 1, 4, 4, None, 0, None) == NULL
    assert f(A, B_, None, None, None, 1, 4, 4, None, 0, None) == NULL
    # small B * D needs a workspace
    assert f(A, B_, None, C, None, 1, 4096, 64, None, 0, None) == WS
    assert f(A, B_, None, C, None, 1, 4096, 64, D_, 100, None) == WS
    # outputs overlapping inputs or each other
    assert f(A, B_, None, A, None, 1, 4096, 64, D_, 1 << 20, None) == ALIAS
    assert f(A, B_, None, C, B_ + 16, 1, 4096, 64, D_, 1 << 20, None) == ALIAS
    assert f(A, B_, None, C, None, 1, 4096, 64, C + 4, 1 << 20, None) == ALIAS
    # empty batch / channels: no-op
    assert f(None, None, None, None, None, 0, 4, 4, None, 0, None) == OK
    assert f(None, None, None, None, None, 3, 4, 0, None, 0, None) == OK


def test_check_log_decay_validation(lib):
    f = lib.cla_check_log_decay
    assert f(A, -1, B_, None) == SHAPE
    assert f(A, 16, None, None) == NULL
    assert f(None, 16, B_, None) == NULL
    assert f(A, 16, B_ + 2, None) == UNSUP        # counts not 4-byte aligned
    assert f(A, 16, A + 8, None) == ALIAS         # counts inside the decays
    assert f(A, 16, A + 60, None) == ALIAS        # overlapping the last value


def test_scan_fwd_noalloc_validation(lib):
    f = lib.cla_scan_fwd_noalloc
    assert f(A, B_, None, C, None, -1, 4, 4, None) == SHAPE
    assert f(A, B_, None, C, None, 1, 4, -4, None) == SHAPE
    assert f(None, B_, None, C, None, 1, 4, 4, None) == NULL
    assert f(A, None, None, C, None, 1, 4, 4, None) == NULL
    assert f(A, B_, None, None, None, 1, 4, 4, None) == NULL
    assert f(A, B_, None, A, None, 1, 4096, 64, None) == ALIAS
    assert f(A, B_, None, C, B_ + 16, 1, 4096, 64, None) == ALIAS
    assert f(A, B_, D_, C, D_, 1, 4096, 64, None) == ALIAS
    assert f(None, None, None, None, None, 0, 4, 4, None) == OK
    assert f(None, None, None, None, None, 3, 4, 0, None) == OK


def test_noalloc_array_covers_every_plan(lib):
    """The fixed array behind cla_scan_fwd_noalloc (256 KiB) holds the largest
    workspace the scan planner asks for: the time axis is split only when
    B * ceil(D / 64) < 512 groups, into at most ceil(512 / groups) segments."""
    worst = 0
    for B in (1, 2, 3, 5, 7, 8):
        for D in (1, 3, 4, 63, 64, 65, 128, 191, 192, 1000, 4096, 32704):
            for T in (1, 127, 128, 129, 4096, 65535, 65536, 1 << 20, 1 << 24):
                worst = max(worst, lib.cla_scan_workspace_bytes(B, T, D))
    assert 0 < worst <= 262144
    assert lib.cla_scan_workspace_bytes(1, 65536, 64) == 511 * 64 * 8


def test_scan_bwd_validation(lib):
    f = lib.cla_scan_bwd
    assert f(A, B_, None, C, None, D_, E, None, 1, -1, 4, None, 0, None) == SHAPE
    for i in range(5):
        args = [A, B_, None, C, None, D_, E, None]
        args[[0, 1, 3, 5, 6][i]] = None
        assert f(*args, 1, 4, 4, None, 0, None) == NULL
    assert f(A, B_, None, C, None, D_, E, None, 1, 4096, 64, None, 0, None) == WS
    assert f(A, B_, None, C, None, C, E, None, 1, 4096, 64, F, 1 << 20, None) == ALIAS
    assert f(A, B_, None, C, None, D_, D_, None, 1, 4096, 64, F, 1 << 20, None) == ALIAS
    assert f(None, None, None, None, None, None, None, None, 0, 9, 9, None, 0, None) == OK


def test_chunk_validation(lib):
    fw = lib.cla_chunk_fwd
    bw = lib.cla_chunk_bwd
    ws = lib.cla_chunk_workspace_bytes
    assert ws(1, 1, 64, 32, 64, 64, 0) == 0          # unsupported head size
    assert fw(A, B_, C, D_, None, E, None, -1, 1, 64, 64, 64, 64, None, 0, None) == SHAPE
    assert fw(A, B_, C, D_, None, E, None, 1, 1, 64, 32, 64, 64, None, 0, None) == UNSUP
    assert fw(A, B_, C, D_, None, E, None, 1, 1, 64, 64, 96, 64, None, 0, None) == UNSUP
    assert fw(A, B_, C, D_, None, E, None, 1, 1, 64, 64, 64, 32, None, 0, None) == UNSUP
    assert fw(None, B_, C, D_, None, E, None, 1, 1, 64, 64, 64, 64, None, 0, None) == NULL
    assert fw(A, B_, C, D_, None, None, None, 1, 1, 64, 64, 64, 64, None, 0, None) == NULL
    assert fw(A, B_, C, D_, None, A, None, 1, 1, 64, 64, 64, 64, F, 1 << 30, None) == ALIAS
    assert fw(None, None, None, None, None, None, None, 0, 4, 64, 64, 64, 64, None, 0, None) == OK
    args = [A, B_, C, D_, None, E, None, F, G, H_, I, None]
    assert bw(*args, 1, 1, 64, 64, 128, 32, None, 0, None) == UNSUP
    for idx in (0, 1, 2, 3, 5, 7, 8, 9, 10):
        a2 = list(args)
        a2[idx] = None
        assert bw(*a2, 1, 1, 64, 64, 64, 64, None, 0, None) == NULL, idx
    a2 = list(args)
    a2[8] = A  # dk aliases q
    assert bw(*a2, 1, 1, 64, 64, 64, 64, J, 1 << 30, None) == ALIAS


def test_chunk_saved_validation(lib):
    # 16 heads of 98304 tokens: 96 backward segments of 16 chunks
    nb = lib.cla_chunk_saved_bytes(1, 16, 98304, 128, 128, 64)
    assert nb == 95 * 16 * 128 * 128 * 4
    # enough heads to fill the GPU without splitting: nothing to save
    assert lib.cla_chunk_saved_bytes(96, 16, 1024, 128, 128, 64) == 0
    assert lib.cla_chunk_saved_bytes(1, 16, 98304, 96, 128, 64) == 0
    assert lib.cla_chunk_saved_bytes(-1, 16, 98304, 128, 128, 64) == 0
    ws = lib.cla_chunk_workspace_bytes(1, 16, 98304, 128, 128, 64, 1)
    f = lib.cla_chunk_fwd_saved
    args = (1, 16, 98304, 128, 128, 64)
    # saved missing or too small
    assert f(A, B_, C, D_, None, E, None, None, 0, *args, F, ws, None) == WS
    assert f(A, B_, C, D_, None, E, None, G, nb - 4, *args, F, ws, None) == WS
    # saved overlapping an input or the output
    assert f(A, B_, C, D_, None, E, None, A, nb, *args, F, ws, None) == ALIAS
    assert f(A, B_, C, D_, None, E, None, E + 64, nb, *args, F, ws, None) == ALIAS
    b = lib.cla_chunk_bwd_saved
    out = (H_, I, J, K, None)
    assert b(A, B_, C, D_, None, E, None, None, 0, *out, *args, F, ws, None) == WS
    assert b(A, B_, C, D_, None, E, None, G, nb - 1, *out, *args, F, ws, None) == WS
    # saved states are an input of the backward: an output may not overlap them
    assert b(A, B_, C, D_, None, E, None, H_, nb, *out, *args, F, ws, None) == ALIAS
    assert b(A, B_, C, D_, None, E, None, G, nb, *out, 1, 16, 98304, 96, 128, 64,
             F, ws, None) == UNSUP


def test_chunk_length_limit(lib):
    # the kernels' grid holds at most 65535 segments along time; backward
    # segments hold at most 16 chunks of 64 tokens: T <= 16 * 65535 * 64
    tmax = 16 * 65535 * 64
    fw = lib.cla_chunk_fwd
    bw = lib.cla_chunk_bwd
    big = 1 << 40  # workspace size large enough to pass the workspace check
    for T, want in ((tmax + 1, UNSUP), (tmax + 64, UNSUP)):
        assert fw(A, B_, C, D_, None, E, None, 1, 1, T, 64, 64, 64, F, big, None) == want
        assert bw(A, B_, C, D_, None, E, None, G, H_, I, J, None, 1, 1, T, 64, 64, 64,
                  K, big, None) == want
    # at the limit the host checks pass (workspace missing is reported next)
    assert fw(A, B_, C, D_, None, E, None, 1, 1, tmax, 64, 64, 64, None, 0, None) == WS
    assert bw(A, B_, C, D_, None, E, None, G, H_, I, J, None, 1, 1, tmax, 64, 64, 64,
              None, 0, None) == WS


def test_gla_validation(lib):
    ws = lib.cla_gla_workspace_bytes
    assert ws(1, 1, 64, 64, 64, 64, 0) == 0                 # the forward needs none
    assert ws(1, 1, 64, 64, 64, 64, 1) > 0
    assert ws(1, 1, 64, 32, 64, 64, 1) == 0                 # unsupported head size
    fw = lib.cla_gla_fwd
    shp = (1, 1, 64, 64, 64, 64)
    assert fw(A, B_, C, D_, None, E, None, -1, 1, 64, 64, 64, 64, None, 0, None) == SHAPE
    assert fw(A, B_, C, D_, None, E, None, 1, 1, 64, 64, 64, 32, None, 0, None) == UNSUP
    assert fw(A, B_, C, D_ + 4, None, E, None, *shp, None, 0, None) == UNSUP  # log decay misaligned
    assert fw(A, B_, C, None, None, E, None, *shp, None, 0, None) == NULL
    assert fw(A, B_, C, D_, None, A, None, *shp, None, 0, None) == ALIAS
    bw = lib.cla_gla_bwd
    need = ws(*shp, 1)
    args = [A, B_, C, D_, None, E, None, F, G, H_, I, None]
    assert bw(*args, *shp, None, 0, None) == WS
    assert bw(*args, *shp, J, need - 16, None) == WS
    for idx in (0, 1, 2, 3, 5, 7, 8, 9, 10):
        a2 = list(args)
        a2[idx] = None
        assert bw(*a2, *shp, J, need, None) == NULL, idx
    a2 = list(args)
    a2[10] = D_  # dlog_decay aliases log_decay
    assert bw(*a2, *shp, J, need, None) == ALIAS
    assert bw(*args, *shp, F, need, None) == ALIAS  # workspace overlaps dq


def test_gla_saved_validation(lib):
    # 16 heads of 98304 tokens: 32 segments of 3 blocks of 16 chunks
    nb = lib.cla_gla_saved_bytes(1, 16, 98304, 128, 128, 64)
    assert nb == 31 * 16 * 128 * 128 * 4
    # 512 sequence-heads fill the GPU without splitting: nothing to save
    assert lib.cla_gla_saved_bytes(32, 16, 4096, 128, 128, 64) == 0
    assert lib.cla_gla_saved_bytes(1, 16, 98304, 96, 128, 64) == 0
    assert lib.cla_gla_saved_bytes(-1, 16, 98304, 128, 128, 64) == 0
    args = (1, 16, 98304, 128, 128, 64)
    wf = lib.cla_gla_workspace_bytes(*args, 0)
    f = lib.cla_gla_fwd_saved
    # saved missing, too small or misaligned
    assert f(A, B_, C, D_, None, E, None, None, 0, *args, F, wf, None) == WS
    assert f(A, B_, C, D_, None, E, None, G, nb - 16, *args, F, wf, None) == WS
    assert f(A, B_, C, D_, None, E, None, G + 4, nb, *args, F, wf, None) == WS
    # saved overlapping an input, the output or the workspace
    assert f(A, B_, C, D_, None, E, None, A, nb, *args, F, wf, None) == ALIAS
    assert f(A, B_, C, D_, None, E, None, E + 64, nb, *args, F, wf, None) == ALIAS
    assert f(A, B_, C, D_, None, E, None, F, nb, *args, F, wf, None) == ALIAS
    wb = lib.cla_gla_workspace_bytes(*args, 1)
    b = lib.cla_gla_bwd_saved
    out = (H_, I, J, K, None)
    assert b(A, B_, C, D_, None, E, None, None, 0, *out, *args, F, wb, None) == WS
    assert b(A, B_, C, D_, None, E, None, G, nb - 16, *out, *args, F, wb, None) == WS
    # saved states are an input of the backward: an output may not overlap them
    assert b(A, B_, C, D_, None, E, None, H_, nb, *out, *args, F, wb, None) == ALIAS
    assert b(A, B_, C, D_, None, E, None, G, nb, *out, 1, 16, 98304, 96, 128, 64,
             F, wb, None) == UNSUP
    # no split: no saved states needed (NULL accepted)
    assert lib.cla_gla_fwd_saved(A, B_, C, D_, None, E, None, None, 0, 1, 1, 0, 64, 64, 64,
                                 None, 0, None) == OK


def test_sscan_validation(lib):
    ck = lib.cla_sscan_ckpt_bytes
    ws = lib.cla_sscan_workspace_bytes
    # checkpoints: the state before every 16th step
    assert ck(2, 100, 64, 16) == 2 * 7 * 64 * 16 * 4
    assert ck(1, 4, 64, 5) == 0 and ck(1, 4, 66, 16) == 0   # N or D unsupported
    # enough (sequence, 64-channel group) units: no time split, no forward workspace
    assert ws(8, 4096, 4096, 16, 0, 0) == 0
    # few units: time is split (4 segments of one 32-step tile here), and the
    # forward keeps each segment's state and decay product
    bdn = 2 * 64 * 16 * 4
    assert ws(2, 100, 64, 16, 0, 0) == 2 * 3 * bdn
    # backward: per-workgroup dB/dC partials, dA per (segment, sequence), and
    # each segment's adjoint and decay product, plus checkpoints and the
    # forward's workspace when the forward's checkpoints are not given
    with_ck = ws(2, 100, 64, 16, 1, 1)
    assert with_ck == 2 * 1 * 100 * 32 * 4 + 4 * bdn + 2 * 4 * bdn
    assert ws(2, 100, 64, 16, 1, 0) == with_ck + ck(2, 100, 64, 16) + 2 * 3 * bdn
    assert ws(2, 0, 64, 16, 1, 1) == 0
    fw = lib.cla_sscan_fwd
    shp = (8, 64, 4096, 16)  # no split
    nows = (None, 0, None)
    assert fw(A, B_, C, D_, E, None, F, None, None, -1, 64, 64, 16, *nows) == SHAPE
    assert fw(A, B_, C, D_, E, None, F, None, None, 8, 64, 4096, 12, *nows) == UNSUP
    assert fw(A, B_, C, D_, E, None, F, None, None, 8, 64, 4094, 16, *nows) == UNSUP
    assert fw(A + 4, B_, C, D_, E, None, F, None, None, *shp, *nows) == UNSUP  # misaligned x
    for idx in (0, 1, 2, 3, 4, 6):
        a2 = [A, B_, C, D_, E, None, F, None, None]
        a2[idx] = None
        assert fw(*a2, *shp, *nows) == NULL, idx
    assert fw(A, B_, C, D_, E, None, A, None, None, *shp, *nows) == ALIAS        # y over x
    assert fw(A, B_, C, D_, E, None, F, None, F + 64, *shp, *nows) == ALIAS      # ckpt over y
    assert fw(None, None, C, None, None, None, None, None, None, 2, 0, 64, 16, *nows) == OK
    # split: the workspace is required, and may not overlap an output
    need = ws(2, 100, 64, 16, 0, 0)
    assert fw(A, B_, C, D_, E, None, F, None, None, 2, 100, 64, 16, None, 0, None) == WS
    assert fw(A, B_, C, D_, E, None, F, None, None, 2, 100, 64, 16, G, need - 16, None) == WS
    assert fw(A, B_, C, D_, E, None, F, None, None, 2, 100, 64, 16, F, need, None) == ALIAS
    bw = lib.cla_sscan_bwd
    shp = (2, 100, 64, 16)
    without = ws(*shp, 1, 0)
    args = [A, B_, C, D_, E, None, None, F, None, G, H_, I, J, K, None]
    assert bw(*args, *shp, None, 0, None) == WS
    assert bw(*args, *shp, L, without - 16, None) == WS
    for idx in (0, 1, 2, 3, 4, 7, 9, 10, 11, 12, 13):
        a2 = list(args)
        a2[idx] = None
        assert bw(*a2, *shp, L, without, None) == NULL, idx
    a2 = list(args)
    a2[9] = F  # dx aliases dy
    assert bw(*a2, *shp, L, without, None) == ALIAS
    assert bw(*args, *shp, G, without, None) == ALIAS  # workspace overlaps dx


def test_stream_probe_rejects_before_launch(lib):
    """The benchmark's streaming probe (a library of its own) loads, exports
    its one call and returns -1 for arguments it does not take, before any
    launch."""
    from chunkwise_linear_attention_amd import build as cbuild
    probe = ctypes.CDLL(cbuild.PROBE_LIB)
    f = probe.cla_probe_stream_3r2w
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    assert f(None, B_, C, D_, E, 8, 16, 4096, None) == -1          # NULL input
    assert f(A, B_, C, D_, None, 8, 16, 4096, None) == -1          # NULL output
    assert f(A, B_, C, D_, E, 8, 16, 4000, None) == -1             # D % 64
    assert f(A, B_, C, D_, E, 1, 16, 64, None) == -1               # groups % 8
    assert f(A, B_, C, D_, E, 0, 16, 4096, None) == -1             # empty
    assert f(A + 4, B_, C, D_, E, 8, 16, 4096, None) == -1         # misaligned
