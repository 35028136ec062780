"""Throughput of the hot path on one MI355X: forward+backward tokens/s, with the
dominant kernel's roofline fraction and the float64 oracle timed on the host
cores beside it.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is the forward and the backward call over one batch of the
workload's synthetic inputs, already resident in HBM.  The default workload
is the diagonal scan B=8, T=16384, D=4096 (fp32).  The chunkwise workloads
(la_const, la_gated, la_long_T*) are selected with --workload.  Prints ONE
JSON line.
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(name):
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_tag, workload, src):
    """HBM bytes per launch measured with rocprofv3 counters and committed
    under profiles/ (the line 'traffic_bytes_per_launch: N' of
    <kernel_tag>_<workload>_traffic.txt); None when absent or when the kernel
    source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel_tag}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != source_hash(src):
        return None
    return float(m.group(1))


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


# ---------------------------------------------------------------------------
# diagonal scan
# ---------------------------------------------------------------------------


def bench_scan(args, torch, cla, wl):
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

    timer = Timer(torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("[bench] warmup done")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step")
    # per-call durations (one kernel each when the time axis is not split)
    f_ms = float(np.mean(timer.time(fwd, args.steps)))
    b_ms = float(np.mean(timer.time(bwd, args.steps)))
    n = B * T * D
    fwd_bytes = pm.scan_bytes_per_elem("fwd") * n
    bwd_bytes = pm.scan_bytes_per_elem("bwd") * n
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
    extra = {"fwd_ms": round(f_ms, 5), "bwd_ms": round(b_ms, 5),
             "fwdbwd_GBps": round((fwd_bytes + bwd_bytes) / (ms_step * 1e-3) / 1e9, 1),
             "workspace_bytes": ws}
    cpu = None
    if args.cpu_baseline:
        cpu = cpu_baseline_scan(inp, B, T, D)
    return dict(value=B * T / (ms_step * 1e-3), ms_per_step=ms_step, dtype="f32",
                config={"workload": wl.name, "B": B, "T": T, "D": D, "tokens_per_step": B * T},
                roofline=roof, cpu_baseline=cpu, extra=extra)


def cpu_baseline_scan(inp, B, T, D):
    """The C oracle (float64 loops, OpenMP over channels) on the whole
    workload, run in blocks of 512 channels so its float64 outputs stay
    bounded in host memory.  The backward reads the oracle's own forward
    output rounded to fp32."""
    from oracle import cref
    cref.build()
    blk = 512
    secs = 0.0
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
    return {"value": round(B * T / secs, 1), "unit": "tokens/s",
            "cores": cref.num_threads(), "kind": "oracle",
            "sample": f"the whole workload (B={B}, T={T}, D={D}), forward+backward, "
                      f"in blocks of {blk} channels: {secs:.2f} s"}


# ---------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="scan_large", choices=sorted(syn.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (the reference "
                         "kernel for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import chunkwise_linear_attention_amd as cla
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = syn.WORKLOADS[args.workload]
    if wl.kind == "scan":
        res = bench_scan(args, torch, cla, wl)
    else:
        raise SystemExit(f"workload {wl.name}: chunkwise bench not available yet")
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
