"""ctypes wrapper over the C oracle loops (oracle/ref.c) -- TEST
INFRASTRUCTURE ONLY.

``build()`` compiles ``ref.c`` into ``oracle/liboracle.so`` with gcc (float64,
OpenMP).  The functions below take the exact device inputs as numpy arrays:
fp32 arrays as float32, bf16 tensors as their uint16 bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle (always recompiles)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
           _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_scan_fwd.argtypes = [p, p, p, p, p] + [i64] * 7
        lib.oracle_scan_bwd.argtypes = [p, p, p, p, p, p, p, p] + [i64] * 7
        lib.oracle_la_fwd.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, p, i64]
        lib.oracle_la_bwd.argtypes = [p] * 12 + [i64, i64, i64, p, i64]
        lib.oracle_gla_fwd.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, p, i64]
        lib.oracle_gla_bwd.argtypes = [p] * 12 + [i64, i64, i64, p, i64]
        lib.oracle_sscan_fwd.argtypes = [p] * 6 + [i64] * 4 + [p, i64, p, p]
        lib.oracle_sscan_bwd.argtypes = [p] * 8 + [i64] * 4 + [p, i64] + [p] * 6
        _lib = lib
    return _lib


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _c(x, dtype):
    return None if x is None else np.ascontiguousarray(x, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def scan_fwd(a, b, h0=None, brange=None, drange=None):
    """a, b: float32 [B, T, D]; h0: float32 [B, D] or None.
    Returns (h, hT) float64 for channels b in brange, d in drange."""
    lib = _load()
    a = _c(a, np.float32)
    b = _c(b, np.float32)
    h0 = _c(h0, np.float32)
    B, T, D = a.shape
    b0, b1 = brange or (0, B)
    d0, d1 = drange or (0, D)
    h = np.empty((b1 - b0, T, d1 - d0))
    hT = np.empty((b1 - b0, d1 - d0))
    lib.oracle_scan_fwd(_ptr(a), _ptr(b), _ptr(h0), _ptr(h), _ptr(hT),
                        B, T, D, b0, b1, d0, d1)
    return h, hT


def scan_bwd(a, h, h0, dh, dhT=None, brange=None, drange=None):
    """a, h, dh: float32 [B, T, D]; h0, dhT: float32 [B, D] or None.
    Returns (da, db, dh0) float64 for the channel block."""
    lib = _load()
    a = _c(a, np.float32)
    h = _c(h, np.float32)
    dh = _c(dh, np.float32)
    h0 = _c(h0, np.float32)
    dhT = _c(dhT, np.float32)
    B, T, D = a.shape
    b0, b1 = brange or (0, B)
    d0, d1 = drange or (0, D)
    da = np.empty((b1 - b0, T, d1 - d0))
    db = np.empty((b1 - b0, T, d1 - d0))
    dh0 = np.empty((b1 - b0, d1 - d0))
    lib.oracle_scan_bwd(_ptr(a), _ptr(h), _ptr(h0), _ptr(dh), _ptr(dhT),
                        _ptr(da), _ptr(db), _ptr(dh0), B, T, D, b0, b1, d0, d1)
    return da, db, dh0


def _heads(heads, B, H):
    if heads is None:
        heads = np.arange(B * H, dtype=np.int64)
    return np.ascontiguousarray(heads, dtype=np.int64)


def la_fwd(q, k, v, l, S0=None, heads=None):
    """q, k: uint16 (bf16 bits) [B, H, T, DK]; v: uint16 [B, H, T, DV];
    l: float32 [B, H, T]; S0: float32 [B, H, DK, DV] or None.
    heads: flat indices b*H + h (default: all).
    Returns (o [n, T, DV], ST [n, DK, DV]) float64."""
    lib = _load()
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    l = _c(l, np.float32)
    S0 = _c(S0, np.float32)
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    hs = _heads(heads, B, H)
    o = np.empty((len(hs), T, DV))
    ST = np.empty((len(hs), DK, DV))
    lib.oracle_la_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(l), _ptr(S0), _ptr(o),
                      _ptr(ST), T, DK, DV, _ptr(hs), len(hs))
    return o, ST


def la_bwd(q, k, v, l, S0, dO, dST=None, heads=None):
    """As ``la_fwd`` plus dO: uint16 [B, H, T, DV] and dST: float32
    [B, H, DK, DV] or None.  Returns (dq, dk, dv, dl, dS0) float64."""
    lib = _load()
    q, k, v, dO = (_c(x, np.uint16) for x in (q, k, v, dO))
    l = _c(l, np.float32)
    S0 = _c(S0, np.float32)
    dST = _c(dST, np.float32)
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    hs = _heads(heads, B, H)
    n = len(hs)
    dq = np.empty((n, T, DK))
    dk = np.empty((n, T, DK))
    dv = np.empty((n, T, DV))
    dl = np.empty((n, T))
    dS0 = np.empty((n, DK, DV))
    lib.oracle_la_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(l), _ptr(S0), _ptr(dO),
                      _ptr(dST), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dl),
                      _ptr(dS0), T, DK, DV, _ptr(hs), n)
    return dq, dk, dv, dl, dS0


def gla_fwd(q, k, v, l, S0=None, heads=None):
    """One decay per key dimension: l is float32 [B, H, T, DK]; the rest as
    ``la_fwd``.  Returns (o [n, T, DV], ST [n, DK, DV]) float64."""
    lib = _load()
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    l = _c(l, np.float32)
    S0 = _c(S0, np.float32)
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    hs = _heads(heads, B, H)
    o = np.empty((len(hs), T, DV))
    ST = np.empty((len(hs), DK, DV))
    lib.oracle_gla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(l), _ptr(S0), _ptr(o),
                       _ptr(ST), T, DK, DV, _ptr(hs), len(hs))
    return o, ST


def gla_bwd(q, k, v, l, S0, dO, dST=None, heads=None):
    """Backward of ``gla_fwd``.  Returns (dq, dk, dv, dl [n, T, DK], dS0)."""
    lib = _load()
    q, k, v, dO = (_c(x, np.uint16) for x in (q, k, v, dO))
    l = _c(l, np.float32)
    S0 = _c(S0, np.float32)
    dST = _c(dST, np.float32)
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    hs = _heads(heads, B, H)
    n = len(hs)
    dq = np.empty((n, T, DK))
    dk = np.empty((n, T, DK))
    dv = np.empty((n, T, DV))
    dl = np.empty((n, T, DK))
    dS0 = np.empty((n, DK, DV))
    lib.oracle_gla_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(l), _ptr(S0), _ptr(dO),
                       _ptr(dST), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dl),
                       _ptr(dS0), T, DK, DV, _ptr(hs), n)
    return dq, dk, dv, dl, dS0


def _chans(chans, Bt, D):
    if chans is None:
        return np.arange(Bt * D, dtype=np.int64)
    return np.ascontiguousarray(chans, dtype=np.int64)


def sscan_fwd(x, delta, A, Bm, Cm, h0=None, chans=None):
    """Selective scan forward on the (batch, channel) units chans (b * D + d;
    default all).  x, delta [Bt, T, D], A [D, N], B, C [Bt, T, N], h0 [Bt, D, N]
    or None, all fp32.  Returns y [nch, T] and hT [nch, N]."""
    lib = _load()
    x, delta, A, Bm, Cm = (_c(v, np.float32) for v in (x, delta, A, Bm, Cm))
    h0 = _c(h0, np.float32)
    Bt, T, D = x.shape
    N = A.shape[1]
    ch = _chans(chans, Bt, D)
    y = np.empty((len(ch), T))
    hT = np.empty((len(ch), N))
    lib.oracle_sscan_fwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(h0),
                         Bt, T, D, N, _ptr(ch), len(ch), _ptr(y), _ptr(hT))
    return y, hT


def sscan_bwd(x, delta, A, Bm, Cm, h0, dy, dhT=None, chans=None):
    """Backward of ``sscan_fwd`` on the units chans.  Returns dx, ddelta
    [nch, T], dA [nch, N] (each unit's own sum over t), dB, dC [Bt, T, N]
    (sums over the listed units), dh0 [nch, N]."""
    lib = _load()
    x, delta, A, Bm, Cm, dy = (_c(v, np.float32) for v in (x, delta, A, Bm, Cm, dy))
    h0, dhT = _c(h0, np.float32), _c(dhT, np.float32)
    Bt, T, D = x.shape
    N = A.shape[1]
    ch = _chans(chans, Bt, D)
    n = len(ch)
    dx = np.empty((n, T))
    dd = np.empty((n, T))
    dA = np.empty((n, N))
    dB = np.empty((Bt, T, N))
    dC = np.empty((Bt, T, N))
    dh0 = np.empty((n, N))
    lib.oracle_sscan_bwd(_ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(h0),
                         _ptr(dy), _ptr(dhT), Bt, T, D, N, _ptr(ch), n, _ptr(dx), _ptr(dd),
                         _ptr(dA), _ptr(dB), _ptr(dC), _ptr(dh0))
    return dx, dd, dA, dB, dC, dh0
