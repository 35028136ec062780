"""Throughput of the hot path on one MI355X: forward+backward tokens/s, with the
dominant kernel's roofline fraction and the float64 oracle timed on the host
cores beside it.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is the forward and the backward call over one batch of the
workload's synthetic inputs, already resident in HBM.  The default workload
is the diagonal scan B=8, T=16384, D=4096 (fp32); the same run also times the
small scan (B=1, T=4096, D=64), the chunkwise workloads (la_const, la_gated,
la_long_T*), the selective scan (sscan_*) and the per-key-dimension decay
workloads (gla_*), each with its roofline and its own oracle baseline, and
reports them under "extra", with streaming ceilings measured on the same GPU.
Any of them can be the headline with --workload.  Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synthetic as syn  # noqa: E402
from chunkwise_linear_attention_amd import perfmodel as pm  # noqa: E402

METRIC = "fwd+bwd tokens/s + % roofline (HBM GB/s for scan, MFMA util chunkwise)"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "chunkwise_linear_attention_amd", "csrc")
# the GPU's clocks settle only after some tens of milliseconds of work
# (measured: about 15 fwd+bwd steps of 2 ms), so every leg warms up for at
# least this long, whatever --warmup says
MIN_WARMUP_S = 0.15


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(name):
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _profile_fields(path, src, keys):
    """Numeric fields `key: value` of a committed counter summary, or None
    when it is absent or the kernel source changed since it was taken."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not h or h.group(1) != source_hash(src):
        return None
    out = {}
    for k in keys:
        m = re.search(rf"^{k}:\s*([0-9.eE+-]+)\s*$", text, re.M)
        if m:
            out[k] = float(m.group(1))
    return out or None


def measured_traffic(kernel_tag, workload, src):
    """HBM bytes per launch measured with rocprofv3 counters and committed
    under profiles/ (the line 'traffic_bytes_per_launch: N' of
    <kernel_tag>_<workload>_traffic.txt); None when absent or when the kernel
    source changed since the counters were taken."""
    f = _profile_fields(os.path.join(PROFILES, f"{kernel_tag}_{workload}_traffic.txt"), src,
                        ["traffic_bytes_per_launch"])
    return None if f is None else f["traffic_bytes_per_launch"]


def measured_mfma(kernel_tag, workload, src):
    """MFMA counters of one kernel from a committed rocprofv3 summary
    (<kernel_tag>_<workload>_mfma.txt): bf16 MFMA flops per launch
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), the MFMA-busy fraction of the SIMDs
    (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs)), and the VALU and
    LDS instruction counts; None when absent or stale."""
    return _profile_fields(os.path.join(PROFILES, f"{kernel_tag}_{workload}_mfma.txt"), src,
                           ["mfma_flops_per_launch", "mfma_busy_frac", "mfma_tflops",
                            "valu_insts_per_launch", "lds_insts_per_launch",
                            "lds_bank_conflict_frac", "wait_inst_any_frac"])


def host_info():
    """What the oracle baseline ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"nproc": os.cpu_count(), "affinity_cpus": aff, "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def oracle_baseline(value, cores, sample):
    d = {"value": round(value, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
         "sample": sample}
    d.update(host_info())
    return d


class Timer:
    """HIP events on torch's current stream, which is where the library
    launches its kernels."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, iters):
        t = self.torch
        starts = [t.cuda.Event(enable_timing=True) for _ in range(iters)]
        ends = [t.cuda.Event(enable_timing=True) for _ in range(iters)]
        for i in range(iters):
            starts[i].record()
            fn()
            ends[i].record()
        t.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def warm_up(torch, step, n_min):
    """Untimed steps: at least n_min of them and at least MIN_WARMUP_S of
    wall time with the GPU busy.  Returns (steps run, seconds)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(max(1, n_min if n == 0 else 2)):
            step()
            n += 1
        torch.cuda.synchronize()
        if n >= n_min and time.perf_counter() - t0 >= MIN_WARMUP_S:
            return n, time.perf_counter() - t0


def timed_steps(torch, step, steps):
    """ms per step over `steps` back-to-back steps, bracketed by events."""
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def library_kernel_times(torch, step, steps):
    """{kernel: (total ms, launches)} from the library's own HIP events
    recorded on the launch stream around every kernel, over `steps` steps."""
    from chunkwise_linear_attention_amd import _lib
    _lib.timing_enable(True)
    try:
        for _ in range(steps):
            step()
        return _lib.timing_read()
    finally:
        _lib.timing_enable(False)


# ---------------------------------------------------------------------------
# diagonal scan
# ---------------------------------------------------------------------------


def bench_scan(args, torch, cla, wl, steps, warmup, cpu=True):
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = wl.make()
    log(f"[bench] inputs for {wl.name} drawn in {time.time() - t0:.1f}s")
    B, T, D = wl.shape["B"], wl.shape["T"], wl.shape["D"]
    g = lambda x: None if x is None else torch.from_numpy(x).to(dev)
    a, b, dh, h0, dhT = g(inp.a), g(inp.b), g(inp.dh), g(inp.h0), g(inp.dhT)
    ws = cla.scan_workspace_bytes(B, T, D)
    wsb = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
    h = torch.empty_like(a)
    hT = torch.empty((B, D), dtype=torch.float32, device=dev)
    da = torch.empty_like(a)
    db = torch.empty_like(a)
    dh0 = torch.empty((B, D), dtype=torch.float32, device=dev)
    L = cla.lib()
    stream = torch.cuda.current_stream(dev).cuda_stream

    def fwd():
        st = L.cla_scan_fwd(a.data_ptr(), b.data_ptr(), h0.data_ptr() if h0 is not None else None,
                            h.data_ptr(), hT.data_ptr(), B, T, D, wsb.data_ptr(), ws, stream)
        if st:
            raise RuntimeError(L.cla_status_string(st))

    def bwd():
        st = L.cla_scan_bwd(a.data_ptr(), h.data_ptr(), h0.data_ptr() if h0 is not None else None,
                            dh.data_ptr(), dhT.data_ptr() if dhT is not None else None,
                            da.data_ptr(), db.data_ptr(), dh0.data_ptr(), B, T, D,
                            wsb.data_ptr(), ws, stream)
        if st:
            raise RuntimeError(L.cla_status_string(st))

    def step():
        fwd()
        bwd()

    nw, ws_s = warm_up(torch, step, warmup)
    ms_step = timed_steps(torch, step, steps)
    log(f"[bench] {wl.name}: timed {steps} steps: {ms_step:.4f} ms/step")
    # per-kernel durations from the library's own HIP events
    table = library_kernel_times(torch, step, steps)
    kernels = {n: {"avg_ms": round(tot / cnt, 5), "launches_per_step": cnt // steps}
               for n, (tot, cnt) in table.items()}
    n = B * T * D
    fwd_bytes = pm.scan_bytes_per_elem("fwd") * n
    bwd_bytes = pm.scan_bytes_per_elem("bwd") * n
    f_ms, b_ms = kernels["scan_fwd"]["avg_ms"], kernels["scan_bwd"]["avg_ms"]
    if b_ms >= f_ms:
        tag, kbytes, kms = "scan_bwd", bwd_bytes, b_ms
    else:
        tag, kbytes, kms = "scan_fwd", fwd_bytes, f_ms
    achieved = kbytes / (kms * 1e-3) / 1e9
    roof = {"kernel": tag, "bound": "hbm", "achieved": round(achieved, 1),
            "peak": pm.PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / pm.PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(tag, wl.name, "scan.hip"),
            "avg_launch_ms": round(kms, 5),
            "algorithmic_bytes_per_launch": kbytes}
    extra = {"fwd_ms": f_ms, "bwd_ms": b_ms, "kernels": kernels,
             "fwdbwd_GBps": round((fwd_bytes + bwd_bytes) / (ms_step * 1e-3) / 1e9, 1),
             "path_roofline_frac": round((fwd_bytes + bwd_bytes) / (pm.PEAK_HBM_GBS * 1e9)
                                         / (ms_step * 1e-3), 4),
             "workspace_bytes": ws, "warmup_steps_run": nw, "warmup_s": round(ws_s, 3)}
    cpu_res = cpu_baseline_scan(inp, B, T, D) if cpu else None
    res = dict(value=B * T / (ms_step * 1e-3), ms_per_step=ms_step, dtype="f32",
               config={"workload": wl.name, "B": B, "T": T, "D": D, "tokens_per_step": B * T},
               roofline=roof, cpu_baseline=cpu_res, extra=extra)
    del a, b, dh, h0, dhT, wsb, h, hT, da, db, dh0
    torch.cuda.empty_cache()
    return res


def cpu_baseline_scan(inp, B, T, D):
    """The C oracle (float64 loops, OpenMP over channels) on the whole
    workload, run in blocks of 512 channels so its float64 outputs stay
    bounded in host memory; a small workload is repeated for >= 1 s.  The
    backward reads the oracle's own forward output rounded to fp32."""
    from oracle import cref
    cref.build()
    blk = 512
    secs, reps = 0.0, 0
    while True:
        for d0 in range(0, D, blk):
            d1 = min(D, d0 + blk)
            t0 = time.time()
            hr, _ = cref.scan_fwd(inp.a, inp.b, inp.h0, drange=(d0, d1))
            secs += time.time() - t0
            hs = np.zeros((B, T, D), dtype=np.float32) if d0 == 0 else hs
            hs[:, :, d0:d1] = hr
            del hr
        for d0 in range(0, D, blk):
            d1 = min(D, d0 + blk)
            t0 = time.time()
            cref.scan_bwd(inp.a, hs, inp.h0, inp.dh, inp.dhT, drange=(d0, d1))
            secs += time.time() - t0
        reps += 1
        if secs >= 1.0:
            break
    del hs
    return oracle_baseline(B * T * reps / secs, cref.num_threads(),
                           f"the whole workload (B={B}, T={T}, D={D}), forward+backward, "
                           f"in blocks of {blk} channels, {reps} time(s): {secs:.2f} s")


def streaming_ceilings(torch):
    """Plain device streams timed on the same GPU: a 1 GiB copy, and the
    diagonal scan forward's mix (two 2 GiB reads, one 2 GiB write, as
    torch.add).  Bytes moved / median of 5 timings."""
    out = {}
    timer = Timer(torch)
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    y.copy_(x)
    ms = float(np.median(timer.time(lambda: y.copy_(x), 5)))
    out["copy_GBps"] = round(2 * x.numel() * 4 / (ms * 1e-3) / 1e9, 1)
    out["copy_bytes"] = 2 * x.numel() * 4
    del x, y
    a = torch.empty(1 << 29, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    c = torch.empty_like(a)
    torch.add(a, b, out=c)
    ms = float(np.median(timer.time(lambda: torch.add(a, b, out=c), 5)))
    out["two_reads_one_write_GBps"] = round(3 * a.numel() * 4 / (ms * 1e-3) / 1e9, 1)
    del a, b, c
    out.update(scan_bwd_mix_ceiling(torch, timer))
    torch.cuda.empty_cache()
    return out


def scan_bwd_mix_ceiling(torch, timer):
    """The diagonal scan backward's traffic without its arithmetic: three
    reads and two writes per element of [8, 16384, 4096] fp32 arrays, in the
    scan kernels' workgroup and lane order (the streaming probe library built
    beside libcla).  Bytes moved / median of 5 timings."""
    import ctypes
    from chunkwise_linear_attention_amd import build as cbuild
    if not os.path.exists(cbuild.PROBE_LIB):
        raise RuntimeError(f"{cbuild.PROBE_LIB} is missing: run the build first")
    lib = ctypes.CDLL(cbuild.PROBE_LIB)
    fn = lib.cla_probe_stream_3r2w
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    B, T, D = 8, 16384, 4096
    xs = [torch.empty(B * T * D, dtype=torch.float32, device="cuda:0") for _ in range(5)]
    for x in xs[:3]:
        x.fill_(0.5)
    st = torch.cuda.current_stream().cuda_stream
    args = [x.data_ptr() for x in xs] + [B, T, D, st]

    def run():
        r = fn(*args)
        if r != 0:
            raise RuntimeError(f"cla_probe_stream_3r2w returned {r}")

    run()
    ms = float(np.median(timer.time(run, 5)))
    del xs
    return {"scan_bwd_mix_GBps": round(20 * B * T * D / (ms * 1e-3) / 1e9, 1),
            "scan_bwd_mix": "3 reads + 2 writes of [8, 16384, 4096] fp32 in the scan "
                            "kernels' order, no arithmetic dependence"}


# ---------------------------------------------------------------------------
# chunkwise linear attention
# ---------------------------------------------------------------------------


def bench_chunk(args, torch, cla, wl, steps, warmup, cpu_heads=0):
    dev = torch.device("cuda:0")
    t0 = time.time()
    ci = wl.make()
    log(f"[bench] inputs for {wl.name} drawn in {time.time() - t0:.1f}s")
    B, H, T, DK, DV = (wl.shape[x] for x in ("B", "H", "T", "DK", "DV"))

    def up(x):
        if x is None:
            return None
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v, l, S0, dO, dST = (up(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    o = torch.empty_like(v)
    ST = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dl = torch.empty_like(l)
    dS0 = torch.empty_like(ST)
    L = cla.lib()
    wsf = cla.chunk_workspace_bytes(B, H, T, DK, DV, False)
    wsb = cla.chunk_workspace_bytes(B, H, T, DK, DV, True)
    ws = torch.empty(max(wsf, wsb, 1), dtype=torch.uint8, device=dev)
    # the training path: the forward saves the states the backward's
    # segments start from (cla_chunk_fwd_saved / cla_chunk_bwd_saved)
    nsv = int(L.cla_chunk_saved_bytes(B, H, T, DK, DV, 64))
    saved = torch.empty(max(nsv, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    P = lambda t: None if t is None else t.data_ptr()

    def fwd():
        st = L.cla_chunk_fwd_saved(P(q), P(k), P(v), P(l), P(S0), P(o), P(ST), P(saved),
                                   saved.numel(), B, H, T, DK, DV, 64, P(ws), ws.numel(), stream)
        if st:
            raise RuntimeError(L.cla_status_string(st))

    def bwd():
        st = L.cla_chunk_bwd_saved(P(q), P(k), P(v), P(l), P(S0), P(dO), P(dST), P(saved),
                                   saved.numel(), P(dq), P(dk), P(dv), P(dl), P(dS0), B, H, T,
                                   DK, DV, 64, P(ws), ws.numel(), stream)
        if st:
            raise RuntimeError(L.cla_status_string(st))

    def step():
        fwd()
        bwd()

    nw, ws_s = warm_up(torch, step, warmup)
    ms_step = timed_steps(torch, step, steps)
    table = library_kernel_times(torch, step, steps)
    units = B * H * T
    kernels = {}
    for name, (tot, cnt) in table.items():
        avg = tot / cnt
        ent = {"avg_ms": round(avg, 5), "launches_per_step": cnt // steps,
               "share": round(tot / sum(x[0] for x in table.values()), 4)}
        if name in ("chunk_fwd", "chunk_dq", "chunk_dkdv"):
            # every token-head once per launch (segment passes cover a
            # fraction and are reported by time only)
            per = pm.chunk_kernel_bytes(name, DK, DV)
            ent["algorithmic_bytes_per_launch"] = per * units
            ent["GBps"] = round(per * units / (avg * 1e-3) / 1e9, 1)
        kernels[name] = ent
    main = {n: e for n, e in kernels.items() if "GBps" in e and not n.endswith("_segments")}
    dom = max(main, key=lambda n: main[n]["avg_ms"] * main[n]["launches_per_step"])
    d = kernels[dom]
    achieved = d["GBps"]
    path_bytes = pm.chunk_bytes_per_token_head(DK, DV, "fwdbwd") * units
    path_flops = pm.chunk_flops_per_token_head(64, DK, DV, "fwdbwd") * units
    t_roof = pm.roofline_seconds(path_bytes, path_flops)
    src_of = lambda n: "chunk.hip" if n in ("chunk_fwd", "chunk_dq") else "chunk_bwd.hip"
    roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": pm.PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / pm.PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(dom, wl.name, src_of(dom)),
            "avg_launch_ms": d["avg_ms"],
            "algorithmic_bytes_per_launch": d["algorithmic_bytes_per_launch"]}
    # MFMA use from rocprofv3 counters (committed summaries), per kernel and
    # over the step: measured bf16 MFMA flops / (step time x 2.5 PFLOP/s)
    mfma = {}
    for n in ("chunk_fwd", "chunk_dq", "chunk_dkdv"):
        c = measured_mfma(n, wl.name, src_of(n))
        if c is not None:
            mfma[n] = c
    mfma_step = None
    if mfma and all(n in mfma for n in ("chunk_fwd", "chunk_dq", "chunk_dkdv")):
        fl = sum(mfma[n]["mfma_flops_per_launch"] * kernels[n]["launches_per_step"] for n in mfma)
        mfma_step = round(fl / (ms_step * 1e-3) / (pm.PEAK_BF16_TFLOPS * 1e12), 4)
    res = {"value": B * T / (ms_step * 1e-3), "ms_per_step": ms_step, "dtype": "bf16",
           "config": {"workload": wl.name, "B": B, "H": H, "T": T, "DK": DK, "DV": DV,
                      "chunk": 64, "tokens_per_step": B * T},
           "roofline": roof,
           "extra": {"kernels": kernels,
                     "path_algorithmic_bytes": path_bytes, "path_algorithmic_flops": path_flops,
                     "path_roofline_frac": round(t_roof / (ms_step * 1e-3), 4),
                     "mfma_util_algorithmic": round(path_flops / (ms_step * 1e-3)
                                                    / (pm.PEAK_BF16_TFLOPS * 1e12), 4),
                     "mfma_util_counters": mfma_step,
                     "mfma_counters": mfma or None,
                     "hbm_GBps_path": round(path_bytes / (ms_step * 1e-3) / 1e9, 1),
                     "workspace_bytes": [wsf, wsb], "saved_state_bytes": nsv,
                     "warmup_steps_run": nw, "warmup_s": round(ws_s, 3),
                     "path": "cla_chunk_fwd_saved + cla_chunk_bwd_saved"}}
    del q, k, v, l, S0, dO, dST, o, ST, dq, dk, dv, dl, dS0, ws, saved
    torch.cuda.empty_cache()
    res["cpu_baseline"] = cpu_baseline_chunk(ci, cpu_heads) if cpu_heads else None
    return res


def cpu_baseline_chunk(ci, nheads):
    """The C oracle (float64 loops, OpenMP over heads), forward then backward,
    on the first `nheads` (batch, head) sequences at full length."""
    from oracle import cref
    cref.build()
    B, H, T, DK = ci.q.shape
    heads = np.arange(min(nheads, B * H), dtype=np.int64)
    t0 = time.time()
    cref.la_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0, heads=heads)
    cref.la_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST, heads=heads)
    secs = time.time() - t0
    frac = len(heads) / (B * H)
    return oracle_baseline(B * T * frac / secs, min(cref.num_threads(), len(heads)),
                           f"{len(heads)} of {B * H} (batch, head) sequences at full length "
                           f"T={T}, forward+backward, {secs:.2f} s; tokens/s scaled by the "
                           "head fraction")


def bench_gla(args, torch, cla, wl, steps, warmup, cpu_heads=0):
    """One decay per key dimension: cla_gla_fwd_saved + cla_gla_bwd_saved per
    step (the training path: the backward starts its segments from the
    forward's saved states; bit-identical to the plain calls)."""
    dev = torch.device("cuda:0")
    t0 = time.time()
    ci = wl.make()
    log(f"[bench] inputs for {wl.name} drawn in {time.time() - t0:.1f}s")
    B, H, T, DK, DV = (wl.shape[x] for x in ("B", "H", "T", "DK", "DV"))

    def up(x):
        if x is None:
            return None
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v, l, S0, dO, dST = (up(x) for x in (ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST))
    o = torch.empty_like(v)
    ST = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dl = torch.empty_like(l)
    dS0 = torch.empty_like(ST)
    L = cla.lib()
    wsf = int(L.cla_gla_workspace_bytes(B, H, T, DK, DV, 64, 0))
    wsb = int(L.cla_gla_workspace_bytes(B, H, T, DK, DV, 64, 1))
    ws = torch.empty(max(wsf, wsb, 1), dtype=torch.uint8, device=dev)
    svb = int(L.cla_gla_saved_bytes(B, H, T, DK, DV, 64))
    saved = torch.empty(max(svb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    P = lambda t: None if t is None else t.data_ptr()

    def fwd():
        st = L.cla_gla_fwd_saved(P(q), P(k), P(v), P(l), P(S0), P(o), P(ST), P(saved),
                                 saved.numel(), B, H, T, DK, DV, 64, P(ws), ws.numel(), stream)
        if st:
            raise RuntimeError(L.cla_status_string(st))

    def bwd():
        st = L.cla_gla_bwd_saved(P(q), P(k), P(v), P(l), P(S0), P(dO), P(dST), P(saved),
                                 saved.numel(), P(dq), P(dk), P(dv), P(dl), P(dS0), B, H, T, DK,
                                 DV, 64, P(ws), ws.numel(), stream)
        if st:
            raise RuntimeError(L.cla_status_string(st))

    def step():
        fwd()
        bwd()

    nw, ws_s = warm_up(torch, step, warmup)
    ms_step = timed_steps(torch, step, steps)
    table = library_kernel_times(torch, step, steps)
    units = B * H * T
    kernels = {}
    total = sum(x[0] for x in table.values())
    for name, (tot, cnt) in table.items():
        avg = tot / cnt
        ent = {"avg_ms": round(avg, 5), "launches_per_step": cnt // steps,
               "share": round(tot / total, 4)}
        if name in ("gla_fwd", "gla_dq", "gla_dkdv"):
            per = pm.gla_kernel_bytes(name, DK, DV)
            ent["algorithmic_bytes_per_launch"] = per * units
            ent["GBps"] = round(per * units / (avg * 1e-3) / 1e9, 1)
        kernels[name] = ent
    main = {n: e for n, e in kernels.items() if "GBps" in e}
    dom = max(main, key=lambda n: main[n]["avg_ms"] * main[n]["launches_per_step"])
    d = kernels[dom]
    path_bytes = pm.gla_bytes_per_token_head(DK, DV, "fwdbwd") * units
    path_flops = pm.gla_flops_per_token_head(64, DK, DV, "fwdbwd") * units
    t_roof = pm.roofline_seconds(path_bytes, path_flops)
    src_of = lambda n: "gla.hip" if n == "gla_fwd" else "gla_bwd.hip"
    roof = {"kernel": dom, "bound": "hbm", "achieved": d["GBps"], "peak": pm.PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(d["GBps"] / pm.PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(dom, wl.name, src_of(dom)),
            "avg_launch_ms": d["avg_ms"],
            "algorithmic_bytes_per_launch": d["algorithmic_bytes_per_launch"]}
    mfma = {}
    for n in ("gla_fwd", "gla_dq", "gla_dkdv"):
        c = measured_mfma(n, wl.name, src_of(n))
        if c is not None:
            mfma[n] = c
    res = {"value": B * T / (ms_step * 1e-3), "ms_per_step": ms_step, "dtype": "bf16",
           "config": {"workload": wl.name, "B": B, "H": H, "T": T, "DK": DK, "DV": DV,
                      "chunk": 64, "tokens_per_step": B * T, "decay": "per key dimension"},
           "roofline": roof,
           "extra": {"kernels": kernels,
                     "path_algorithmic_bytes": path_bytes, "path_algorithmic_flops": path_flops,
                     "path_roofline_frac": round(t_roof / (ms_step * 1e-3), 4),
                     "mfma_util_algorithmic": round(path_flops / (ms_step * 1e-3)
                                                    / (pm.PEAK_BF16_TFLOPS * 1e12), 4),
                     "mfma_counters": mfma or None,
                     "hbm_GBps_path": round(path_bytes / (ms_step * 1e-3) / 1e9, 1),
                     "workspace_bytes": [wsf, wsb], "saved_bytes": svb,
                     "warmup_steps_run": nw, "warmup_s": round(ws_s, 3),
                     "path": "cla_gla_fwd_saved + cla_gla_bwd_saved"}}
    del q, k, v, l, S0, dO, dST, o, ST, dq, dk, dv, dl, dS0, ws, saved
    torch.cuda.empty_cache()
    res["cpu_baseline"] = cpu_baseline_gla(ci, cpu_heads) if cpu_heads else None
    return res


def cpu_baseline_gla(ci, nheads):
    """The C oracle for one decay per key dimension, forward then backward, on
    the first `nheads` (batch, head) sequences at full length."""
    from oracle import cref
    cref.build()
    B, H, T, DK = ci.q.shape
    heads = np.arange(min(nheads, B * H), dtype=np.int64)
    t0 = time.time()
    cref.gla_fwd(ci.q, ci.k, ci.v, ci.l, ci.S0, heads=heads)
    cref.gla_bwd(ci.q, ci.k, ci.v, ci.l, ci.S0, ci.dO, ci.dST, heads=heads)
    secs = time.time() - t0
    frac = len(heads) / (B * H)
    return oracle_baseline(B * T * frac / secs, min(cref.num_threads(), len(heads)),
                           f"{len(heads)} of {B * H} (batch, head) sequences at full length "
                           f"T={T}, forward+backward, {secs:.2f} s; tokens/s scaled by the "
                           "head fraction")


def bench_sscan(args, torch, cla, wl, steps, warmup, cpu_channels=0):
    """Selective scan, N entries per channel: cla_sscan_fwd (with checkpoints)
    + cla_sscan_bwd per step."""
    dev = torch.device("cuda:0")
    t0 = time.time()
    ci = wl.make()
    log(f"[bench] inputs for {wl.name} drawn in {time.time() - t0:.1f}s")
    B, T, D, N = (wl.shape[k] for k in ("B", "T", "D", "N"))
    up = lambda v: None if v is None else torch.from_numpy(v).to(dev)
    x, dl, A, Bm, Cm, h0, dy, dhT = (up(v) for v in (ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0,
                                                     ci.dy, ci.dhT))
    y = torch.empty_like(x)
    hT = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    dx, dd = torch.empty_like(x), torch.empty_like(x)
    dA = torch.empty((D, N), dtype=torch.float32, device=dev)
    dB, dC = torch.empty_like(Bm), torch.empty_like(Cm)
    dh0 = torch.empty_like(hT)
    L = cla.lib()
    ck = torch.empty(int(L.cla_sscan_ckpt_bytes(B, T, D, N)) // 4, dtype=torch.float32,
                     device=dev)
    wsf = int(L.cla_sscan_workspace_bytes(B, T, D, N, 0, 0))
    wsb = int(L.cla_sscan_workspace_bytes(B, T, D, N, 1, 1))
    ws = torch.empty(max(wsf, wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    P = lambda t: None if t is None else t.data_ptr()

    def fwd():
        st = L.cla_sscan_fwd(P(x), P(dl), P(A), P(Bm), P(Cm), P(h0), P(y), P(hT), P(ck),
                             B, T, D, N, P(ws), ws.numel(), stream)
        if st:
            raise RuntimeError(L.cla_status_string(st))

    def bwd():
        st = L.cla_sscan_bwd(P(x), P(dl), P(A), P(Bm), P(Cm), P(h0), P(ck), P(dy), P(dhT), P(dx),
                             P(dd), P(dA), P(dB), P(dC), P(dh0), B, T, D, N, P(ws), wsb, stream)
        if st:
            raise RuntimeError(L.cla_status_string(st))

    def step():
        fwd()
        bwd()

    nw, ws_s = warm_up(torch, step, warmup)
    ms_step = timed_steps(torch, step, steps)
    table = library_kernel_times(torch, step, steps)
    elems = B * T * D * N
    kernels = {}
    total = sum(x_[0] for x_ in table.values())
    for name, (tot, cnt) in table.items():
        avg = tot / cnt
        ent = {"avg_ms": round(avg, 5), "launches_per_step": cnt // steps,
               "share": round(tot / total, 4)}
        if name in ("sscan_fwd", "sscan_bwd"):
            dirn = "fwd" if name == "sscan_fwd" else "bwd"
            ops = pm.sscan_ops_per_element(dirn) * elems
            by = pm.sscan_bytes(B, T, D, N, dirn)
            ent["algorithmic_ops_per_launch"] = ops
            ent["Tops"] = round(ops / (avg * 1e-3) / 1e12, 3)
            ent["algorithmic_bytes_per_launch"] = by
            ent["GBps"] = round(by / (avg * 1e-3) / 1e9, 1)
        kernels[name] = ent
    main = {n: e for n, e in kernels.items() if "Tops" in e}
    dom = max(main, key=lambda n: main[n]["avg_ms"])
    d = kernels[dom]
    path_ops = pm.sscan_ops_per_element("fwdbwd") * elems
    path_bytes = pm.sscan_bytes(B, T, D, N, "fwdbwd")
    t_roof = max(path_ops / (pm.PEAK_VALU_TOPS * 1e12), path_bytes / (pm.PEAK_HBM_GBS * 1e9))
    roof = {"kernel": dom, "bound": "alu", "achieved": d["Tops"], "peak": round(pm.PEAK_VALU_TOPS, 2),
            "unit": "Top/s (fp32 VALU lane-ops, exp = 4)", "frac": round(d["Tops"] / pm.PEAK_VALU_TOPS, 4),
            "traffic": measured_traffic(dom, wl.name, "sscan.hip"),
            "avg_launch_ms": d["avg_ms"],
            "algorithmic_ops_per_launch": d["algorithmic_ops_per_launch"]}
    res = {"value": B * T / (ms_step * 1e-3), "ms_per_step": ms_step, "dtype": "f32",
           "config": {"workload": wl.name, "B": B, "T": T, "D": D, "N": N,
                      "tokens_per_step": B * T},
           "roofline": roof,
           "extra": {"kernels": kernels, "path_algorithmic_ops": path_ops,
                     "path_algorithmic_bytes": path_bytes,
                     "path_roofline_frac": round(t_roof / (ms_step * 1e-3), 4),
                     "hbm_GBps_path": round(path_bytes / (ms_step * 1e-3) / 1e9, 1),
                     "checkpoint_bytes": ck.numel() * 4, "workspace_bytes": [wsf, wsb],
                     "warmup_steps_run": nw, "warmup_s": round(ws_s, 3),
                     "path": "cla_sscan_fwd (checkpoints) + cla_sscan_bwd"}}
    del x, dl, A, Bm, Cm, dy, y, hT, dx, dd, dA, dB, dC, dh0, ck, ws
    torch.cuda.empty_cache()
    res["cpu_baseline"] = cpu_baseline_sscan(ci, cpu_channels) if cpu_channels else None
    return res


def cpu_baseline_sscan(ci, nch):
    """The C oracle (float64 loops, OpenMP over channels), forward then
    backward, on the first `nch` (sequence, channel) units at full length."""
    from oracle import cref
    cref.build()
    B, T, D = ci.x.shape
    chans = np.arange(min(nch, B * D), dtype=np.int64)
    t0 = time.time()
    cref.sscan_fwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, chans=chans)
    cref.sscan_bwd(ci.x, ci.delta, ci.A, ci.Bm, ci.Cm, ci.h0, ci.dy, ci.dhT, chans=chans)
    secs = time.time() - t0
    frac = len(chans) / (B * D)
    return oracle_baseline(B * T * frac / secs, cref.num_threads(),
                           f"{len(chans)} of {B * D} (sequence, channel) units at full length "
                           f"T={T}, N={ci.A.shape[1]}, forward+backward, {secs:.2f} s; tokens/s "
                           "scaled by the channel fraction")


CHUNK_EXTRAS = ("la_const", "la_gated") + tuple(f"la_long_T{t}" for t in syn.LONG_T)
GLA_EXTRAS = ("gla_T4096", "gla_long_T98304")
SSCAN_EXTRAS = ("sscan_mamba", "sscan_b1")


def _summary(r, keys=("path_roofline_frac",)):
    s = {"tokens_per_s": round(r["value"], 1), "ms_per_step": round(r["ms_per_step"], 4),
         "dtype": r["dtype"], "config": r["config"], "roofline": r["roofline"],
         "cpu_baseline": r["cpu_baseline"],
         "kernels": {n: e["avg_ms"] for n, e in r["extra"]["kernels"].items()}}
    for k in keys:
        if k in r["extra"]:
            s[k] = r["extra"][k]
    return s


def oracle_threads():
    from oracle import cref
    cref.build()
    return cref.num_threads()


def main():
    global MIN_WARMUP_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help=f"untimed steps per workload (at least {MIN_WARMUP_S} s of them "
                         "are run in any case)")
    ap.add_argument("--workload", default="scan_large", choices=sorted(syn.WORKLOADS))
    ap.add_argument("--min-warmup-s", type=float, default=MIN_WARMUP_S,
                    help="least wall time of untimed steps per workload (0 for profiler runs)")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--no-chunk-extras", action="store_true",
                    help="with the scan workload, skip the other workloads")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="chunkwise/GLA workloads: sequences the oracle baseline runs "
                         "(default: one per oracle thread)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (the reference "
                         "kernel for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    MIN_WARMUP_S = max(0.0, args.min_warmup_s)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import chunkwise_linear_attention_amd as cla
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    nthr = oracle_threads() if args.cpu_baseline else 0
    cpu_heads = (args.cpu_heads or nthr) if args.cpu_baseline else 0
    wl = syn.WORKLOADS[args.workload]
    if wl.kind == "scan":
        res = bench_scan(args, torch, cla, wl, args.steps, args.warmup, cpu=args.cpu_baseline)
        if wl.name == "scan_large" and not args.no_chunk_extras:
            ex = res["extra"]
            ex["streaming_ceilings"] = sc = streaming_ceilings(torch)
            # the headline kernel against the same traffic without arithmetic
            if res["roofline"]["kernel"] == "scan_bwd":
                sc["scan_bwd_over_mix_ceiling"] = round(
                    res["roofline"]["achieved"] / sc["scan_bwd_mix_GBps"], 4)
            # the small scan (one channel group, time split into segments):
            # launch latency dominates, so more steps are timed
            r = bench_scan(args, torch, cla, syn.WORKLOADS["scan_small"], max(200, args.steps),
                           args.warmup, cpu=args.cpu_baseline)
            ex["scan_small"] = _summary(r, ("path_roofline_frac", "fwdbwd_GBps"))
            # the matrix-state rows of the hot path, measured in the same run
            chunk = {}
            for name in CHUNK_EXTRAS:
                r = bench_chunk(args, torch, cla, syn.WORKLOADS[name], max(3, args.steps // 2),
                                args.warmup, cpu_heads=cpu_heads)
                chunk[name] = _summary(r, ("path_roofline_frac", "mfma_util_algorithmic",
                                           "mfma_util_counters", "mfma_counters"))
                log(f"[bench] {name}: {r['ms_per_step']:.3f} ms/step")
            longs = [chunk[f"la_long_T{t}"]["tokens_per_s"] for t in syn.LONG_T]
            ex["chunkwise"] = chunk
            for name in SSCAN_EXTRAS:
                wsc = syn.WORKLOADS[name]
                r = bench_sscan(args, torch, cla, wsc, max(3, args.steps // 2), args.warmup,
                                cpu_channels=(wsc.shape["B"] * wsc.shape["D"] // 8)
                                if args.cpu_baseline else 0)
                ex.setdefault("selective_scan", {})[name] = _summary(r)
                log(f"[bench] {name}: {r['ms_per_step']:.3f} ms/step")
            for name in GLA_EXTRAS:
                r = bench_gla(args, torch, cla, syn.WORKLOADS[name], max(3, args.steps // 2),
                              args.warmup, cpu_heads=cpu_heads)
                ex.setdefault("gla", {})[name] = _summary(r, ("path_roofline_frac",
                                                              "mfma_util_algorithmic",
                                                              "mfma_counters"))
                log(f"[bench] {name}: {r['ms_per_step']:.3f} ms/step")
            ex["la_long_T_flatness_min_over_max"] = round(min(longs) / max(longs), 4)
    elif wl.kind == "sscan":
        # the oracle runs the whole workload (every channel): a few seconds
        res = bench_sscan(args, torch, cla, wl, args.steps, args.warmup,
                          cpu_channels=wl.shape["B"] * wl.shape["D"] if args.cpu_baseline else 0)
    elif wl.kind == "gla":
        res = bench_gla(args, torch, cla, wl, args.steps, args.warmup, cpu_heads=cpu_heads)
    else:
        res = bench_chunk(args, torch, cla, wl, args.steps, args.warmup, cpu_heads=cpu_heads)
    if args.copy_probe:
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        res["extra"]["copy_probe_bytes"] = x.numel() * 4
    out = {"metric": METRIC, "value": round(res["value"], 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(res["ms_per_step"], 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"],
           "data": "synthetic", "config": res["config"], "roofline": res["roofline"],
           "cpu_baseline": res["cpu_baseline"], "extra": res["extra"]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
