"""ctypes loader for libcla.so (the C ABI declared in include/cla.h).

Argument marshalling only.  The library must have been built in-tree
(``python -m chunkwise_linear_attention_amd.build``); a missing library is a
hard error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcla.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "cla.h")

CLA_OK = 0
STATUS_NAMES = {0: "CLA_OK", 1: "CLA_ERR_NULL_ARG", 2: "CLA_ERR_BAD_SHAPE",
                3: "CLA_ERR_UNSUPPORTED", 4: "CLA_ERR_WORKSPACE",
                5: "CLA_ERR_ALIAS", 6: "CLA_ERR_HIP"}


class ClaError(RuntimeError):
    """A libcla entry point returned a non-zero status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.fn = fn
        self.status = status


_lib = None
p = ctypes.c_void_p
i64 = ctypes.c_int64
sz = ctypes.c_size_t

SIGNATURES = {
    "cla_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "cla_version": ([], ctypes.c_char_p),
    "cla_check_log_decay": ([p, i64, p, p], ctypes.c_int),
    "cla_scan_workspace_bytes": ([i64, i64, i64], sz),
    "cla_scan_fwd": ([p, p, p, p, p, i64, i64, i64, p, sz, p], ctypes.c_int),
    "cla_scan_fwd_noalloc": ([p, p, p, p, p, i64, i64, i64, p], ctypes.c_int),
    "cla_scan_bwd": ([p, p, p, p, p, p, p, p, i64, i64, i64, p, sz, p], ctypes.c_int),
    "cla_chunk_workspace_bytes": ([i64, i64, i64, i64, i64, i64, ctypes.c_int], sz),
    "cla_chunk_fwd": ([p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, p, sz, p],
                      ctypes.c_int),
    "cla_chunk_bwd": ([p] * 12 + [i64] * 6 + [p, sz, p], ctypes.c_int),
    "cla_chunk_saved_bytes": ([i64] * 6, sz),
    "cla_chunk_fwd_saved": ([p] * 8 + [sz] + [i64] * 6 + [p, sz, p], ctypes.c_int),
    "cla_chunk_bwd_saved": ([p] * 8 + [sz] + [p] * 5 + [i64] * 6 + [p, sz, p], ctypes.c_int),
    "cla_gla_workspace_bytes": ([i64, i64, i64, i64, i64, i64, ctypes.c_int], sz),
    "cla_gla_fwd": ([p] * 7 + [i64] * 6 + [p, sz, p], ctypes.c_int),
    "cla_gla_bwd": ([p] * 12 + [i64] * 6 + [p, sz, p], ctypes.c_int),
    "cla_gla_saved_bytes": ([i64] * 6, sz),
    "cla_gla_fwd_saved": ([p] * 8 + [sz] + [i64] * 6 + [p, sz, p], ctypes.c_int),
    "cla_gla_bwd_saved": ([p] * 8 + [sz] + [p] * 5 + [i64] * 6 + [p, sz, p], ctypes.c_int),
    "cla_sscan_ckpt_bytes": ([i64] * 4, sz),
    "cla_sscan_workspace_bytes": ([i64] * 4 + [ctypes.c_int] * 2, sz),
    "cla_sscan_fwd": ([p] * 9 + [i64] * 4 + [p, sz, p], ctypes.c_int),
    "cla_sscan_bwd": ([p] * 15 + [i64] * 4 + [p, sz, p], ctypes.c_int),
    "cla_timing_enable": ([ctypes.c_int], ctypes.c_int),
    "cla_timing_read": ([p, p, p, ctypes.c_int], ctypes.c_int),
}


def timing_enable(on: bool) -> None:
    lib().cla_timing_enable(1 if on else 0)


def timing_read(max_kernels: int = 32) -> dict:
    """{kernel name: (total ms, launches)} since the last read (synchronizes)."""
    names = (ctypes.c_char_p * max_kernels)()
    tot = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int64 * max_kernels)()
    n = lib().cla_timing_read(names, tot, cnt, max_kernels)
    if n < 0:
        raise ClaError("cla_timing_read", -n, "event query failed")
    return {names[i].decode(): (tot[i], cnt[i]) for i in range(min(n, max_kernels))}


def header_symbols() -> list[str]:
    """Function names declared in include/cla.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cla_[a-z_0-9]+)\s*\(", text)))


def lib():
    """Load libcla.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libcla.so not found at {LIB_PATH}; build it with "
                "`python -m chunkwise_linear_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != CLA_OK:
        msg = lib().cla_status_string(status).decode()
        raise ClaError(fn, status, msg)
