"""ctypes binding of ``libkda_probe.so`` (``include/kda_probe.h``): HBM
streaming probes used by the benchmark to state the achievable ceiling and
by the counter runs as a kernel of known traffic.  Measurement only; the
decode step never calls them.

    python -m hybrid_linear_attention_kda_amd.probe --sweep [--json FILE]

runs the ceiling sweep on ``cuda:0`` (in place, read only, write only and
copy; 256 / 512 / 1024 threads per workgroup; 1, 2 or 4 16-byte chunks per
lane; one workgroup per tile or a persistent grid; 34 launches of 128 MiB,
as the decode launches one per layer, or one launch over all 4.25 GiB) and
prints one table row per shape, timed with HIP events on the launch stream.
"""
from __future__ import annotations

import ctypes
import os

#: the built probe library (see ``build.py``)
LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda_probe.so")

#: every symbol ``include/kda_probe.h`` declares
EXPORTS = ("kda_probe_rmw", "kda_probe_copy", "kda_probe_stream")

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
    i = ctypes.c_int
    lib.kda_probe_stream.argtypes = [i, i, i, i, vp, vp, sz, ctypes.c_float, vp]
    lib.kda_probe_stream.restype = i
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


KINDS = {0: "in place", 1: "read only", 2: "write only", 3: "copy"}


def sweep(chunk_bytes: int = 128 << 20, layers: int = 34, reps: int = 10, warmup: int = 2,
          kinds=(0, 1, 2, 3), threads=(256, 512, 1024), chunks=(1, 2, 4), persistent=(0, 1),
          launches=("per layer", "one")):
    """Time every probe shape over `layers` distinct chunks of `chunk_bytes`.
    Returns a list of dicts; GB/s counts the bytes read plus written."""
    import torch
    lib = load()
    total = chunk_bytes * layers
    src = torch.ones(total // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.ones_like(src)
    stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    rows = []
    for kind in kinds:
        moved = 2 if kind in (0, 3) else 1
        for nt in threads:
            for apl in chunks:
                for pers in persistent:
                    for how in launches:
                        n = layers if how == "per layer" else 1
                        size = total // n

                        def run():
                            for c in range(n):
                                a = ctypes.c_void_p(src.data_ptr() + c * size)
                                b = a if kind == 0 else ctypes.c_void_p(dst.data_ptr() + c * size)
                                _check("kda_probe_stream",
                                       lib.kda_probe_stream(kind, nt, apl, pers, a, b, size, 1.0, sp))

                        with torch.cuda.stream(stream):
                            for _ in range(warmup):
                                run()
                            s0 = torch.cuda.Event(enable_timing=True)
                            s1 = torch.cuda.Event(enable_timing=True)
                            s0.record(stream)
                            for _ in range(reps):
                                run()
                            s1.record(stream)
                            s1.synchronize()
                        sec = s0.elapsed_time(s1) / 1e3
                        rows.append({"kind": KINDS[kind], "threads": nt, "chunks_per_lane": apl,
                                     "persistent": bool(pers), "launches": how, "launch_bytes": size,
                                     "GBps": moved * total * reps / sec / 1e9,
                                     "us_per_launch": sec / (reps * n) * 1e6})
                        print(f"{KINDS[kind]:10s} {nt:5d} x {apl} {'persistent' if pers else 'one-shot  '} "
                              f"{how:9s} {rows[-1]['us_per_launch']:9.2f} us/launch {rows[-1]['GBps']:8.1f} GB/s",
                              flush=True)
    del src, dst
    torch.cuda.empty_cache()
    return rows


if __name__ == "__main__":
    import argparse
    import json
    ap = argparse.ArgumentParser(description="HBM streaming probe sweep (one GPU)")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--chunk-mib", type=int, default=128,
                    help="bytes per launch of the per-layer form (34 launches), MiB")
    ap.add_argument("--kinds", default="0,1,2,3", help="comma-separated kinds: 0 in place, 1 read, 2 write, 3 copy")
    ap.add_argument("--threads", default="256,512,1024")
    ap.add_argument("--chunks", default="1,2,4")
    ap.add_argument("--launches", default="per layer,one")
    ap.add_argument("--persistent", default="0,1", help="comma-separated: 0 one workgroup per tile, 1 grid-stride")
    ap.add_argument("--json", default=None, help="also write the rows to this file")
    a = ap.parse_args()
    if a.sweep:
        ints = lambda v: tuple(int(x) for x in v.split(","))  # noqa: E731
        out = sweep(chunk_bytes=a.chunk_mib << 20, reps=a.reps, kinds=ints(a.kinds), threads=ints(a.threads),
                    chunks=ints(a.chunks), persistent=ints(a.persistent), launches=tuple(a.launches.split(",")))
        if a.json:
            with open(a.json, "w") as f:
                json.dump(out, f, indent=1)
