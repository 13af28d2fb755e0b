"""Build ``libkda.so`` (the gfx950 HIP library behind ``include/kda.h``) and
``libkda_probe.so`` (the measurement probes behind ``include/kda_probe.h``).

    python -m hybrid_linear_attention_kda_amd.build

Compiles ``csrc/kda_kernels.hip``, ``csrc/kda_prefill.hip`` and ``csrc/kda_api.cpp``, and separately
``csrc/kda_probe.hip``, with hipcc for gfx950 only.  Packed-FP32
instructions are switched off for device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libkda.so")
SOURCES = [os.path.join(CSRC, "kda_kernels.hip"), os.path.join(CSRC, "kda_prefill.hip"),
           os.path.join(CSRC, "kda_api.cpp")]
HEADERS = [os.path.join(INCLUDE, "kda.h"), os.path.join(CSRC, "kda_launch.h"), os.path.join(CSRC, "kda_device.h")]
PROBE_LIBRARY = os.path.join(PKG, "libkda_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "kda_probe.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(sources: list[str], output: str, extra: list[str] | None, verbose: bool) -> str:
    tmp = output + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra or []), f"-I{INCLUDE}", f"-I{CSRC}", *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(tmp, output)
    return output


def build(output: str = LIBRARY, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile the decode library to ``output`` and the probe library beside
    the package; returns the decode library's path."""
    _compile(SOURCES, output, extra, verbose)
    _compile(PROBE_SOURCES, PROBE_LIBRARY, None, verbose)
    return output


def is_stale(path: str = LIBRARY) -> bool:
    if not os.path.exists(path) or not os.path.exists(PROBE_LIBRARY):
        return True
    t = min(os.path.getmtime(path), os.path.getmtime(PROBE_LIBRARY))
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS + PROBE_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
