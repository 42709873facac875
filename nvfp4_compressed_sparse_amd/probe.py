"""ctypes binding of libmla_probe.so (include/mla_probe.h): achievable-rate probes that the benchmark runs
beside the decode (streaming read, row gather, MFMA loop).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

from .build import PROBE_LIB, build

EXPORTS = ["mla_probe_stream_read", "mla_probe_row_gather", "mla_probe_mfma", "mla_probe_mfma_flops"]

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB):
            build()
        L = ctypes.CDLL(PROBE_LIB)
        P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        for name, res, args in (("mla_probe_stream_read", ctypes.c_int, [P, i64, P, i32, P]),
                                ("mla_probe_row_gather", ctypes.c_int, [P, P, i64, i32, P, i32, P]),
                                ("mla_probe_mfma", ctypes.c_int, [i32, i32, P, i32, P]),
                                ("mla_probe_mfma_flops", i64, [i32, i32])):
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _ok(name, st):
    if st != 0:
        raise RuntimeError(f"{name} failed with status {st}")


def stream_read(src, sink, workgroups, stream):
    _ok("mla_probe_stream_read", lib().mla_probe_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                                             sink.data_ptr(), workgroups, stream))


def row_gather(pool, addr16, row_bytes, sink, workgroups, stream):
    _ok("mla_probe_row_gather", lib().mla_probe_row_gather(pool.data_ptr(), addr16.data_ptr(), addr16.numel(),
                                                           row_bytes, sink.data_ptr(), workgroups, stream))


def mfma(bf16, iters, out, workgroups, stream):
    _ok("mla_probe_mfma", lib().mla_probe_mfma(int(bool(bf16)), iters, out.data_ptr(), workgroups, stream))


def mfma_flops(iters, workgroups):
    return lib().mla_probe_mfma_flops(iters, workgroups)
