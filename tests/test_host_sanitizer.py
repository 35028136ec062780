"""The C ABI's argument validation under AddressSanitizer and UBSan (CPU).

api.cpp and timing.cpp (the host layer: validation, planning, timing hooks)
are compiled for the host with -fsanitize=address and -fsanitize=undefined,
each flag given to the host compile only (-Xarch_host), linked with the
library's other objects unchanged, and the boundary checks of
test_boundary.py are run against that copy in a child process with every GPU
hidden and the ASan runtime preloaded.  Any sanitizer report fails the test.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "chunkwise_linear_attention_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SOURCES = ("api.cpp", "timing.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_validation_layer_under_asan_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("no hipcc or ASan runtime in this image")
    from chunkwise_linear_attention_amd import build as b
    others = [os.path.join(b.OBJ, os.path.basename(s) + ".o") for s in b.sources()
              if os.path.basename(s) not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in others):
        b.build()
    objs = []
    for name in HOST_SOURCES:
        obj = str(tmp_path / (name + ".o"))
        cmd = [HIPCC, *b.FLAGS, "-O1", "-g", *SAN, "-c", os.path.join(b.CSRC, name), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        objs.append(obj)
    lib = str(tmp_path / "libcla_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=" + b.ARCH, "-shared", "-fPIC", "-o", lib, *objs,
                        *others, *SAN, "-shared-libsan"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "not instrumented"

    env = dict(os.environ)
    env.update({"CLA_BOUNDARY_GPU_HIDDEN": "1", "HIP_VISIBLE_DEVICES": "",
                "ROCR_VISIBLE_DEVICES": "", "CUDA_VISIBLE_DEVICES": "",
                "CLA_BOUNDARY_LIB": lib, "LD_PRELOAD": rt,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    print(out[-3000:])
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out
