"""ctypes binding of ``libkda_probe.so`` (``include/kda_probe.h``): HBM
streaming probes used by the benchmark to state the achievable ceiling and
by the counter runs as a kernel of known traffic.  Measurement only; the
decode step never calls them."""
from __future__ import annotations

import ctypes
import os

#: the built probe library (see ``build.py``)
LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda_probe.so")

#: every symbol ``include/kda_probe.h`` declares
EXPORTS = ("kda_probe_rmw", "kda_probe_copy")

_LIB = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m hybrid_linear_attention_kda_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.kda_probe_rmw.argtypes = [vp, sz, ctypes.c_float, vp]
    lib.kda_probe_rmw.restype = ctypes.c_int
    lib.kda_probe_copy.argtypes = [vp, vp, sz, vp]
    lib.kda_probe_copy.restype = ctypes.c_int
    _LIB = lib
    return lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise RuntimeError(f"{fn} failed with status {rc}")


def kda_probe_rmw(buf, scale: float = 1.0, stream=None):
    """In-place read-modify-write of a contiguous f32 device tensor."""
    s = ctypes.c_void_p(stream.cuda_stream if stream is not None else 0)
    _check("kda_probe_rmw", load().kda_probe_rmw(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                                 float(scale), s))


def kda_probe_copy(src, dst, stream=None):
    """dst = src for two contiguous device tensors of equal size."""
    assert src.numel() * src.element_size() == dst.numel() * dst.element_size()
    s = ctypes.c_void_p(stream.cuda_stream if stream is not None else 0)
    _check("kda_probe_copy", load().kda_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                                   src.numel() * src.element_size(), s))
