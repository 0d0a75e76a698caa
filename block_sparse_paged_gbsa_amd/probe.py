"""ctypes binding of libgbsa_probe.so (include/gbsa_probe.h): HBM ceilings for the benchmark.

Argument marshalling only; the probes are HIP kernels. Loading fails loudly when the library
has not been built.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgbsa_probe.so")
EXPORTED = ("gbsa_probe_gather", "gbsa_probe_stream")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_sparse_paged_gbsa_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        lib.gbsa_probe_gather.argtypes = [vp, vp, vp, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int64, vp, vp]
        lib.gbsa_probe_gather.restype = ctypes.c_int
        lib.gbsa_probe_stream.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp]
        lib.gbsa_probe_stream.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(fn, code):
    if code != 0:
        raise RuntimeError(f"{fn} failed with code {code}")


def gather(key, value, slice_offsets, row_bytes: int, row_stride: int, sink, stream) -> None:
    _check("gbsa_probe_gather", load().gbsa_probe_gather(
        key.data_ptr(), value.data_ptr(), slice_offsets.data_ptr(), slice_offsets.numel(),
        row_bytes, row_stride, sink.data_ptr(), stream.cuda_stream))


def stream_read(src, nbytes: int, grid: int, sink, stream) -> None:
    _check("gbsa_probe_stream", load().gbsa_probe_stream(src.data_ptr(), nbytes, grid,
                                                         sink.data_ptr(), stream.cuda_stream))
