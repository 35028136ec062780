"""Build libcla.so, the HIP library behind the C ABI in include/cla.h.

Compiles every source under csrc/ for gfx950 with hipcc (in parallel, one
object per source) and links them into chunkwise_linear_attention_amd/libcla.so;
also builds the benchmark's streaming probe (probe/libstreamprobe.so).
Always recompiles.  Usage: ``python -m chunkwise_linear_attention_amd.build``.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return obj, out


PROBE_SRC = os.path.join(HERE, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(HERE, "probe", "libstreamprobe.so")


def build_probe() -> str:
    """The benchmark's streaming probe (probe/stream_probe.hip), a library of
    its own that only bench.py loads."""
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        results = list(ex.map(_compile, sources()))
    for _, out in results:
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_probe()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
