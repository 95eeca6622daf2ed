"""ctypes binding of libpa_probe.so (include/pa_probe.h): the streaming-read and matrix-core
probes the benchmark measures its ceilings with.  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa_probe.so")
SIGNATURES = {
    "pa_probe_read": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]),
    "pa_probe_mfma": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]),
}
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def read(buf, blocks: int, sink):
    """Enqueue one streaming read of the whole uint8 device tensor `buf`."""
    st = load().pa_probe_read(buf.data_ptr(), buf.numel(), blocks, sink.data_ptr(), _stream())
    if st != 0:
        raise RuntimeError(f"pa_probe_read: {st}")


def mfma(blocks: int, iters: int, shape: int, sink):
    """Enqueue one matrix-core loop; returns its flop count."""
    st = load().pa_probe_mfma(blocks, iters, shape, sink.data_ptr(), _stream())
    if st != 0:
        raise RuntimeError(f"pa_probe_mfma: {st}")
    return blocks * 4 * iters * 8 * (16384 if shape == 16 else 32768)
