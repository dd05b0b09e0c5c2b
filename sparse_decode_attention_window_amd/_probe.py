"""ctypes binding of libkvsel_probe.so, the benchmark's HBM stream probe (a
measurement aid, not part of the method): non-temporal 16-byte read or copy
streams over a fixed grid, used to state the rate a call of a given size can
reach.  Raises ImportError when the library has not been built."""
from __future__ import annotations

import ctypes
import os

from ._lib import KvselError, _ptr, _stream

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(_PKG, "libkvsel_probe.so")
PROBE_READ, PROBE_COPY, PROBE_BLOCKS = 0, 1, 2048
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_PATH):
            raise ImportError(f"{PROBE_PATH} is missing: build it with "
                              "python -m sparse_decode_attention_window_amd.build")
        l = ctypes.CDLL(PROBE_PATH)
        l.kvsel_probe_stream.restype = ctypes.c_int
        l.kvsel_probe_stream.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_void_p]
        _lib = l
    return _lib


def probe_stream(mode: int, src, dst, nbytes: int, stream=None) -> None:
    """READ: dst gets PROBE_BLOCKS 16-byte XOR folds of src; COPY: dst = src."""
    st = lib().kvsel_probe_stream(int(mode), _ptr(src), _ptr(dst), int(nbytes), _stream(stream))
    if st != 0:
        raise KvselError(f"kvsel_probe_stream: status {st}")
