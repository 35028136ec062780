"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random numbers
and casts them (fp32 by round-to-nearest-even, bf16 by round-to-nearest-even
of the fp32 value).  Both the GPU path and the float64 oracle read what it
returns, so they see bit-identical inputs.

Generator: numpy PCG64.  Each tensor of a workload gets its own child of
``SeedSequence(seed)`` in a fixed order, and each block of ``_BLOCK`` elements
of a tensor gets its own grandchild, so the values do not depend on how many
threads draw them.  Normal draws are float32 (``standard_normal(dtype=
float32)``) times a float32 scale; uniform draws are float64.

Workloads (sizes as used by the bench and the full-size tests):

* ``scan_small``  -- diagonal scan, B=1, T=4096, D=64, delta ~ U(1e-3, 0.1),
  a = exp(-delta), b ~ N(0,1), h0 = 0, upstream gradient ~ N(0,1).
* ``scan_large``  -- diagonal scan, B=8, T=16384, D=4096, delta ~ U(1e-4, 0.5),
  b ~ N(0,1), h0 ~ N(0,1), upstream gradient ~ N(0,1).
* ``la_const``    -- chunkwise linear attention, B=4, H=16, T=8192, dk=dv=64,
  q, k, v ~ N(0,1)/8, per-head constant decay 1 - 2^-(5 + 8h/H), dO ~ N(0,1).
* ``la_gated``    -- B=2, H=32, T=32768, dk=128, dv=64, q, k ~ N(0,1)/sqrt(128),
  v ~ N(0,1), log a = -softplus(N(0,1)) * 0.1, S0 ~ N(0,1) * 0.1, dO ~ N(0,1).
* ``la_long_T``   -- H=16, dk=dv=128, T in {1024, 4096, 16384, 65536, 98304},
  B = 98304 // T, q, k ~ N(0,1)/sqrt(128), v ~ N(0,1), log a = -1e-5 or -5 with
  probability 1/2 each (i.i.d.), dO ~ N(0,1).
* ``sscan_mamba`` -- selective scan with N state entries per channel, at the
  size of one Mamba-2.8B layer on 8 sequences: B=8, T=4096 (32,768 tokens),
  D=5120 channels, N=16; x, B, C, dy ~ N(0,1), delta log-uniform in
  [1e-3, 1e-1], A[d, n] = -(n + 1), no h0.
* ``sscan_b1``    -- the same draws for one sequence of 32,768 tokens and
  D=2048 channels (32 channel groups: time is split into segments).
* ``gla_T4096``   -- one decay per key dimension, B=32, H=16, T=4096,
  dk=dv=128, q, k ~ N(0,1)/sqrt(128), v ~ N(0,1), log a[d] = logsigmoid(x)/16
  with x ~ N(0,1) per (token, dimension), S0 = none, dO ~ N(0,1).
* ``gla_long_T98304`` -- the same draws at B=1, H=16, T=98304 (16
  sequence-heads: the sequence is split into segments).
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_BLOCK = 1 << 22
_THREADS = 8


# ---------------------------------------------------------------------------
# casts
# ---------------------------------------------------------------------------


def _elementwise(fn, x: np.ndarray, dtype) -> np.ndarray:
    """fn applied to blocks of the flattened x by a thread pool (numpy's
    ufuncs release the GIL); the result does not depend on the split."""
    x = np.ascontiguousarray(x)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=dtype)
    n = flat.size
    nblocks = max(1, (n + _BLOCK - 1) // _BLOCK)

    def work(i):
        lo, hi = i * _BLOCK, min(n, (i + 1) * _BLOCK)
        out[lo:hi] = fn(flat[lo:hi])

    if nblocks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nblocks)))
    return out.reshape(x.shape)


def _bf16_round_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16
    bit patterns.  Inputs must be finite."""
    return _elementwise(_bf16_round_bits, np.asarray(x, dtype=np.float32), np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------------------
# block-parallel, thread-count-independent drawing
# ---------------------------------------------------------------------------


def _draw(seed_seq: np.random.SeedSequence, n: int, kind: str, p=()) -> np.ndarray:
    """Draw n values; kind 'normal32' (float32), 'uniform64' (float64, p=(lo,hi)),
    'coin' (bool, probability 1/2)."""
    nblocks = max(1, (n + _BLOCK - 1) // _BLOCK)
    kids = seed_seq.spawn(nblocks)
    dtype = {"normal32": np.float32, "uniform64": np.float64, "coin": np.bool_}[kind]
    out = np.empty(n, dtype=dtype)

    def work(i):
        lo = i * _BLOCK
        hi = min(n, lo + _BLOCK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        if kind == "normal32":
            g.standard_normal(out=out[lo:hi], dtype=np.float32)
        elif kind == "uniform64":
            out[lo:hi] = g.uniform(p[0], p[1], size=hi - lo)
        else:
            out[lo:hi] = g.integers(0, 2, size=hi - lo, dtype=np.uint8).astype(np.bool_)

    if nblocks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nblocks)))
    return out


def _normal_f32(ss, shape, scale=1.0):
    x = _draw(ss, int(np.prod(shape)), "normal32").reshape(shape)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _normal_bf16(ss, shape, scale=1.0):
    return bf16_bits_from_f32(_normal_f32(ss, shape, scale))


# ---------------------------------------------------------------------------
# diagonal scan inputs
# ---------------------------------------------------------------------------


@dataclass
class ScanInputs:
    a: np.ndarray            # [B, T, D] float32
    b: np.ndarray            # [B, T, D] float32
    h0: np.ndarray | None    # [B, D] float32
    dh: np.ndarray           # [B, T, D] float32 (upstream gradient of h)
    dhT: np.ndarray | None   # [B, D] float32 (upstream gradient of h_T)


def scan_inputs(B, T, D, seed, delta=(1e-3, 0.1), h0=False, dhT=False,
                a_const=None) -> ScanInputs:
    """a = exp(-delta), delta ~ U(delta); b, dh ~ N(0,1); h0, dhT ~ N(0,1) when
    requested.  ``a_const`` replaces every decay by that constant (special
    cases a = 1 and a = 0)."""
    ss = np.random.SeedSequence(seed).spawn(5)
    n = B * T * D
    if a_const is None:
        d = _draw(ss[0], n, "uniform64", delta)
        a = np.exp(-d).astype(np.float32).reshape(B, T, D)
        del d
    else:
        a = np.full((B, T, D), a_const, dtype=np.float32)
    b = _normal_f32(ss[1], (B, T, D))
    h0v = _normal_f32(ss[2], (B, D)) if h0 else None
    dh = _normal_f32(ss[3], (B, T, D))
    dhTv = _normal_f32(ss[4], (B, D)) if dhT else None
    return ScanInputs(a, b, h0v, dh, dhTv)


# ---------------------------------------------------------------------------
# chunkwise linear attention inputs
# ---------------------------------------------------------------------------


@dataclass
class ChunkInputs:
    q: np.ndarray            # [B, H, T, DK] uint16 (bf16 bits)
    k: np.ndarray            # [B, H, T, DK] uint16
    v: np.ndarray            # [B, H, T, DV] uint16
    l: np.ndarray            # [B, H, T] float32 log decay ([B, H, T, DK]: per key dim)
    S0: np.ndarray | None    # [B, H, DK, DV] float32
    dO: np.ndarray           # [B, H, T, DV] uint16
    dST: np.ndarray | None   # [B, H, DK, DV] float32


def chunk_inputs(B, H, T, DK, DV, seed, qk_scale=1.0, v_scale=1.0,
                 decay="softplus", S0_scale=None, dST_scale=None) -> ChunkInputs:
    """decay: 'softplus' -> l = -softplus(N(0,1)) * 0.1;
    'head_const' -> l[b,h,t] = fp32(log(1 - 2^-(5 + 8h/H)));
    'mix' -> l = -1e-5 or -5 with probability 1/2 each;
    'zero' -> l = 0 (no decay); ('const', x) -> l = x everywhere;
    ('resets', p) -> the softplus decays with each step replaced, with
    probability p, by l = -inf (a_t = 0: the state is cleared before the
    step's write)."""
    ss = np.random.SeedSequence(seed).spawn(7)
    q = _normal_bf16(ss[0], (B, H, T, DK), qk_scale)
    k = _normal_bf16(ss[1], (B, H, T, DK), qk_scale)
    v = _normal_bf16(ss[2], (B, H, T, DV), v_scale)
    if decay == "softplus":
        x = _draw(ss[3], B * H * T, "normal32").astype(np.float64)
        l = (-np.logaddexp(0.0, x) * 0.1).astype(np.float32).reshape(B, H, T)
    elif decay == "head_const":
        lam = 1.0 - 2.0 ** (-(5.0 + 8.0 * np.arange(H) / H))
        l = np.broadcast_to(np.log(lam).astype(np.float32)[None, :, None],
                            (B, H, T)).copy()
    elif decay == "mix":
        c = _draw(ss[3], B * H * T, "coin").reshape(B, H, T)
        l = np.where(c, np.float32(-5.0), np.float32(-1e-5)).astype(np.float32)
    elif decay == "zero":
        l = np.zeros((B, H, T), dtype=np.float32)
    elif isinstance(decay, tuple) and decay[0] == "const":
        l = np.full((B, H, T), decay[1], dtype=np.float32)
    elif isinstance(decay, tuple) and decay[0] == "resets":
        x = _draw(ss[3], B * H * T, "normal32").astype(np.float64)
        l = (-np.logaddexp(0.0, x) * 0.1).astype(np.float32).reshape(B, H, T)
        u = _draw(ss[3].spawn(1)[0], B * H * T, "uniform64", (0.0, 1.0)).reshape(B, H, T)
        l[u < decay[1]] = -np.inf
    else:
        raise ValueError(f"unknown decay kind {decay!r}")
    S0 = None if S0_scale is None else _normal_f32(ss[4], (B, H, DK, DV), S0_scale)
    dO = _normal_bf16(ss[5], (B, H, T, DV))
    dST = None if dST_scale is None else _normal_f32(ss[6], (B, H, DK, DV), dST_scale)
    return ChunkInputs(q, k, v, l, S0, dO, dST)


def gla_inputs(B, H, T, DK, DV, seed, qk_scale=None, v_scale=1.0,
               decay="logsigmoid", S0_scale=None, dST_scale=None) -> ChunkInputs:
    """Inputs with one log decay per key dimension, l [B, H, T, DK] fp32.
    q, k ~ N(0,1) * qk_scale (default 1/sqrt(DK)), v ~ N(0,1) * v_scale, dO ~
    N(0,1), all bf16.  decay: 'logsigmoid' -> l = logsigmoid(x) / 16 with x ~
    N(0,1) (a sigmoid gate raised to the power 1/16); ('logsigmoid', tau) ->
    logsigmoid(x) / tau; ('const', c) -> l = c everywhere; ('uniform', lo, hi)
    -> l ~ U(lo, hi)."""
    if qk_scale is None:
        qk_scale = 1.0 / math.sqrt(DK)
    ss = np.random.SeedSequence(seed).spawn(7)
    q = _normal_bf16(ss[0], (B, H, T, DK), qk_scale)
    k = _normal_bf16(ss[1], (B, H, T, DK), qk_scale)
    v = _normal_bf16(ss[2], (B, H, T, DV), v_scale)
    n = B * H * T * DK
    if decay == "logsigmoid" or (isinstance(decay, tuple) and decay[0] == "logsigmoid"):
        tau = 16.0 if decay == "logsigmoid" else float(decay[1])
        x = _draw(ss[3], n, "normal32")
        l = _elementwise(lambda y: (-np.logaddexp(0.0, -y.astype(np.float64)) / tau)
                         .astype(np.float32), x, np.float32).reshape(B, H, T, DK)
    elif isinstance(decay, tuple) and decay[0] == "const":
        l = np.full((B, H, T, DK), decay[1], dtype=np.float32)
    elif isinstance(decay, tuple) and decay[0] == "uniform":
        l = _draw(ss[3], n, "uniform64", (decay[1], decay[2])).astype(np.float32)
        l = l.reshape(B, H, T, DK)
    else:
        raise ValueError(f"unknown decay kind {decay!r}")
    S0 = None if S0_scale is None else _normal_f32(ss[4], (B, H, DK, DV), S0_scale)
    dO = _normal_bf16(ss[5], (B, H, T, DV))
    dST = None if dST_scale is None else _normal_f32(ss[6], (B, H, DK, DV), dST_scale)
    return ChunkInputs(q, k, v, l, S0, dO, dST)


@dataclass
class SScanInputs:
    x: np.ndarray            # [B, T, D] float32
    delta: np.ndarray        # [B, T, D] float32 (step sizes, > 0)
    A: np.ndarray            # [D, N] float32
    Bm: np.ndarray           # [B, T, N] float32
    Cm: np.ndarray           # [B, T, N] float32
    h0: np.ndarray | None    # [B, D, N] float32
    dy: np.ndarray           # [B, T, D] float32 (upstream gradient of y)
    dhT: np.ndarray | None   # [B, D, N] float32 (upstream gradient of h_T)


def sscan_inputs(B, T, D, N, seed, delta=("loguniform", 1e-3, 1e-1), A="s4d",
                 h0_scale=None, dhT_scale=None) -> SScanInputs:
    """Selective-scan inputs.  x, B, C, dy ~ N(0,1).  delta: ('loguniform', lo,
    hi) -> exp(U(log lo, log hi)) per (batch, token, channel).  A: 's4d' ->
    A[d, n] = -(n + 1) (the real diagonal initialisation Mamba-1 starts from);
    ('uniform', lo, hi) -> U(lo, hi) per (channel, entry); ('const', c).
    h0, dhT ~ N(0,1) * scale when a scale is given."""
    ss = np.random.SeedSequence(seed).spawn(8)
    n = B * T * D
    x = _normal_f32(ss[0], (B, T, D))
    if delta[0] == "loguniform":
        u = _draw(ss[1], n, "uniform64", (math.log(delta[1]), math.log(delta[2])))
        dl = _elementwise(lambda v: np.exp(v).astype(np.float32), u, np.float32)
        dl = dl.reshape(B, T, D)
        del u
    else:
        raise ValueError(f"unknown delta kind {delta!r}")
    if A == "s4d":
        Am = np.tile(-np.arange(1, N + 1, dtype=np.float32), (D, 1))
    elif A[0] == "uniform":
        Am = _draw(ss[2], D * N, "uniform64", (A[1], A[2])).astype(np.float32).reshape(D, N)
    elif A[0] == "const":
        Am = np.full((D, N), A[1], dtype=np.float32)
    else:
        raise ValueError(f"unknown A kind {A!r}")
    Bm = _normal_f32(ss[3], (B, T, N))
    Cm = _normal_f32(ss[4], (B, T, N))
    h0 = None if h0_scale is None else _normal_f32(ss[5], (B, D, N), h0_scale)
    dy = _normal_f32(ss[6], (B, T, D))
    dhT = None if dhT_scale is None else _normal_f32(ss[7], (B, D, N), dhT_scale)
    return SScanInputs(x, dl, Am, Bm, Cm, h0, dy, dhT)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------


@dataclass
class Workload:
    name: str
    kind: str                 # "scan" or "chunk"
    shape: dict
    make: object = field(repr=False)

    @property
    def tokens(self) -> int:
        return self.shape["B"] * self.shape["T"]


def _scan_small():
    return scan_inputs(1, 4096, 64, 1001, delta=(1e-3, 0.1))


def _scan_large():
    return scan_inputs(8, 16384, 4096, 1002, delta=(1e-4, 0.5), h0=True)


def _la_const():
    return chunk_inputs(4, 16, 8192, 64, 64, 1003, qk_scale=1 / 8, v_scale=1 / 8,
                        decay="head_const")


def _la_gated(dST=False):
    return chunk_inputs(2, 32, 32768, 128, 64, 1004, qk_scale=1 / math.sqrt(128),
                        decay="softplus", S0_scale=0.1,
                        dST_scale=0.1 if dST else None)


LONG_T = (1024, 4096, 16384, 65536, 98304)


def _la_long(T):
    i = LONG_T.index(T)
    return chunk_inputs(98304 // T, 16, T, 128, 128, 1050 + i,
                        qk_scale=1 / math.sqrt(128), decay="mix")


def _sscan_mamba():
    return sscan_inputs(8, 4096, 5120, 16, 1070)


def _sscan_b1():
    return sscan_inputs(1, 32768, 2048, 16, 1071)


def _gla_train():
    return gla_inputs(32, 16, 4096, 128, 128, 1060, decay="logsigmoid")


def _gla_long():
    return gla_inputs(1, 16, 98304, 128, 128, 1061, decay="logsigmoid")


WORKLOADS = {
    "scan_small": Workload("scan_small", "scan", dict(B=1, T=4096, D=64), _scan_small),
    "scan_large": Workload("scan_large", "scan", dict(B=8, T=16384, D=4096), _scan_large),
    "la_const": Workload("la_const", "chunk",
                         dict(B=4, H=16, T=8192, DK=64, DV=64), _la_const),
    "la_gated": Workload("la_gated", "chunk",
                         dict(B=2, H=32, T=32768, DK=128, DV=64), _la_gated),
}
WORKLOADS["sscan_mamba"] = Workload("sscan_mamba", "sscan",
                                    dict(B=8, T=4096, D=5120, N=16), _sscan_mamba)
WORKLOADS["sscan_b1"] = Workload("sscan_b1", "sscan",
                                 dict(B=1, T=32768, D=2048, N=16), _sscan_b1)
WORKLOADS["gla_T4096"] = Workload("gla_T4096", "gla",
                                  dict(B=32, H=16, T=4096, DK=128, DV=128), _gla_train)
WORKLOADS["gla_long_T98304"] = Workload("gla_long_T98304", "gla",
                                        dict(B=1, H=16, T=98304, DK=128, DV=128), _gla_long)
for _T in LONG_T:
    WORKLOADS[f"la_long_T{_T}"] = Workload(
        f"la_long_T{_T}", "chunk", dict(B=98304 // _T, H=16, T=_T, DK=128, DV=128),
        (lambda T=_T: _la_long(T)))
