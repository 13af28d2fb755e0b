"""Double-precision CPU oracle for the KDA decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the CPU-baseline leg of the benchmark may import this module.  The GPU
library never calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``kda_oracle.c`` (plain C, IEEE double, OpenMP over
independent (stream, head) units).  This module builds it with gcc, loads it
with ctypes and marshals numpy float64 arrays.  The sources each routine
follows are cited in the C file:

* "GLM-5.3 deep dive" (gangliao.me), 8.2.3 Eq. 1 and 8.2.6: gated delta rule
  in fade / predict / correct / read order;
* same page, 8.2.4: short causal convolution (kernel 4) with SiLU, L2 norm;
* "At the 262k cap the DSA indexer costs 12x the sparse MLA it selects for",
  "Geometry": depthwise conv, kernel 4, three cached taps;
* "GLM-5.3 deep dive" 8.2.3 (the forget gate as fla computes it) and 8.2.4
  (write strength, gated RMSNorm on the output).

Parity pins for every routine live in ``tests/oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "kda_oracle.c")
LIBRARY = os.path.join(HERE, "libkda_oracle.so")

#: epsilon of the L2 norm, "GLM-5.3 deep dive" 8.2.6 implementation notes.
L2NORM_EPS = 1e-6
#: epsilon of the gated RMSNorm, "GLM-5.3 deep dive" 8.2.4 implementation notes.
RMSNORM_EPS = 1e-5
#: gate forms, "GLM-5.3 deep dive" 8.2.3: bounded sigmoid (GLM-5.3-Flash, lower
#: bound -5) and fla's default softplus form.
GATE_BOUNDED, GATE_SOFTPLUS = 0, 1

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile ``source`` into the shared library ``output`` with gcc."""
    tmp = f"{output}.tmp{os.getpid()}"      # per process: parallel test workers may build at once
    cmd = ["gcc", *_CFLAGS, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


_P = ctypes.POINTER(ctypes.c_double)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


class Oracle:
    """ctypes handle on one build of the C oracle (the real one or a test mutant)."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = LIBRARY
            if (not os.path.exists(path)
                    or os.path.getmtime(path) < os.path.getmtime(SOURCE)):
                build()
        self.path = path
        lib = ctypes.CDLL(path)
        i, d, p = ctypes.c_int, ctypes.c_double, _P
        lib.kda_oracle_conv_silu.argtypes = [i, p, p, p, p, p]
        lib.kda_oracle_conv_silu.restype = None
        lib.kda_oracle_l2norm.argtypes = [i, p, d, d, p]
        lib.kda_oracle_l2norm.restype = None
        lib.kda_oracle_delta_step.argtypes = [i, i, p, p, p, p, p, d, p]
        lib.kda_oracle_delta_step.restype = None
        lib.kda_oracle_decode_step.argtypes = [i, i, i, p, p, p, p, p, p, p, d, d, p]
        lib.kda_oracle_decode_step.restype = i
        lib.kda_oracle_recurrent_step.argtypes = [i, i, i, p, p, p, p, d, d, p]
        lib.kda_oracle_recurrent_step.restype = i
        lib.kda_oracle_max_threads.argtypes = []
        lib.kda_oracle_max_threads.restype = i
        lib.kda_oracle_gate.argtypes = [i, p, d, p, i, d, p]
        lib.kda_oracle_gate.restype = None
        lib.kda_oracle_beta.argtypes = [i, p, p]
        lib.kda_oracle_beta.restype = None
        lib.kda_oracle_gated_rmsnorm.argtypes = [i, p, p, p, d, p]
        lib.kda_oracle_gated_rmsnorm.restype = None
        lib.kda_oracle_decode_step_gated.argtypes = [i, i, i, p, p, p, p, p, p, p, p, p, i, d, d, d, p]
        lib.kda_oracle_decode_step_gated.restype = i
        lib.kda_oracle_layer_step.argtypes = [i, i, i, p, p, p, p, p, p, p, p, p, i, d, d, d, p, p, d, p]
        lib.kda_oracle_layer_step.restype = i
        lib.kda_oracle_decode_multi.argtypes = [i, i, i, i, p, p, p, p, p, p, p, d, d, p]
        lib.kda_oracle_decode_multi.restype = i
        lib.kda_oracle_sequence_gated.argtypes = [i, i, i, i, p, p, p, p, p, p, p, p, p, i, d, d, d, p]
        lib.kda_oracle_sequence_gated.restype = i
        self.lib = lib

    def max_threads(self) -> int:
        return int(self.lib.kda_oracle_max_threads())

    # -- single routines ----------------------------------------------------
    def conv_silu(self, x, w, cs_in):
        """x [C], w [C,4], cs_in [3,C] -> (z [C], cs_out [3,C])."""
        x, w, cs_in = _f64(x), _f64(w), _f64(cs_in)
        C = x.shape[0]
        assert w.shape == (C, 4) and cs_in.shape == (3, C)
        z = np.empty(C)
        cs_out = np.empty((3, C))
        self.lib.kda_oracle_conv_silu(C, _ptr(x), _ptr(w), _ptr(cs_in), _ptr(cs_out), _ptr(z))
        return z, cs_out

    def l2norm(self, x, eps=L2NORM_EPS, scale=1.0):
        x = _f64(x)
        out = np.empty_like(x)
        self.lib.kda_oracle_l2norm(x.shape[0], _ptr(x), float(eps), float(scale), _ptr(out))
        return out

    def delta_step(self, S, q, k, v, alpha, beta):
        """S [dk,dv]; q,k,alpha [dk]; v [dv] -> (S_new, o [dv]).  Inputs untouched."""
        S = _f64(S).copy()
        dk, dv = S.shape
        q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
        assert q.shape == (dk,) and k.shape == (dk,) and alpha.shape == (dk,) and v.shape == (dv,)
        o = np.empty(dv)
        self.lib.kda_oracle_delta_step(dk, dv, _ptr(S), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), float(beta), _ptr(o))
        return S, o

    # -- whole step ---------------------------------------------------------
    def decode_step(self, S, x, w, cs, alpha, beta, scale, eps=L2NORM_EPS):
        """One fused step.  Shapes: S [M,H,D,D], x [M,3,H*D], w [3*H*D,4],
        cs [M,3,3*H*D], alpha [M,H,D], beta [M,H].
        Returns (S_new, cs_new, o [M,H,D]); inputs are not modified."""
        S = _f64(S).copy()
        M, H, D, D2 = S.shape
        assert D == D2
        x, w, cs = _f64(x), _f64(w), _f64(cs)
        alpha, beta = _f64(alpha), _f64(beta)
        assert x.shape == (M, 3, H * D) and w.shape == (3 * H * D, 4)
        assert cs.shape == (M, 3, 3 * H * D)
        assert alpha.shape == (M, H, D) and beta.shape == (M, H)
        cs_out = np.empty_like(cs)
        o = np.empty((M, H, D))
        rc = self.lib.kda_oracle_decode_step(M, H, D, _ptr(S), _ptr(x), _ptr(w), _ptr(cs),
                                             _ptr(cs_out), _ptr(alpha), _ptr(beta),
                                             float(scale), float(eps), _ptr(o))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_decode_step failed ({rc})")
        return S, cs_out, o

    def recurrent_step(self, S, qkv, alpha, beta, scale, eps=L2NORM_EPS):
        """Recurrent part from post-conv q|k|v [M,3,H*D]. Returns (S_new, o)."""
        S = _f64(S).copy()
        M, H, D, _ = S.shape
        qkv, alpha, beta = _f64(qkv), _f64(alpha), _f64(beta)
        assert qkv.shape == (M, 3, H * D)
        o = np.empty((M, H, D))
        rc = self.lib.kda_oracle_recurrent_step(M, H, D, _ptr(S), _ptr(qkv), _ptr(alpha),
                                                _ptr(beta), float(scale), float(eps), _ptr(o))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_recurrent_step failed ({rc})")
        return S, o


    # -- gate, write strength, output norm ------------------------------------
    def gate(self, f, A_log, dt_bias, kind=GATE_BOUNDED, lower_bound=-5.0):
        """One head: f, dt_bias [D], A_log scalar -> alpha [D]."""
        f, b = _f64(f), _f64(dt_bias)
        assert f.shape == b.shape and f.ndim == 1
        out = np.empty_like(f)
        self.lib.kda_oracle_gate(f.shape[0], _ptr(f), float(A_log), _ptr(b), int(kind),
                                 float(lower_bound), _ptr(out))
        return out

    def beta(self, logit):
        logit = _f64(logit)
        out = np.empty_like(logit)
        self.lib.kda_oracle_beta(logit.size, _ptr(logit), _ptr(out))
        return out

    def gated_rmsnorm(self, o, g, w, eps=RMSNORM_EPS):
        """One head: o, g, w [D] -> y [D]."""
        o, g, w = _f64(o), _f64(g), _f64(w)
        assert o.shape == g.shape == w.shape and o.ndim == 1
        y = np.empty_like(o)
        self.lib.kda_oracle_gated_rmsnorm(o.shape[0], _ptr(o), _ptr(g), _ptr(w), float(eps), _ptr(y))
        return y

    def decode_step_gated(self, S, x, w, cs, f, A_log, dt_bias, beta_logit, scale,
                          kind=GATE_BOUNDED, lower_bound=-5.0, eps=L2NORM_EPS):
        """The fused step with raw gate inputs: f [M,H*D], A_log [H],
        dt_bias [H*D], beta_logit [M,H]; the rest as decode_step.
        Returns (S_new, cs_new, o)."""
        S = _f64(S).copy()
        M, H, D, _ = S.shape
        x, w, cs = _f64(x), _f64(w), _f64(cs)
        f, A_log, dt_bias, beta_logit = _f64(f), _f64(A_log), _f64(dt_bias), _f64(beta_logit)
        assert f.shape == (M, H * D) and A_log.shape == (H,) and dt_bias.shape == (H * D,)
        assert beta_logit.shape == (M, H) and x.shape == (M, 3, H * D)
        cs_out = np.empty_like(cs)
        o = np.empty((M, H, D))
        rc = self.lib.kda_oracle_decode_step_gated(M, H, D, _ptr(S), _ptr(x), _ptr(w), _ptr(cs),
                                                   _ptr(cs_out), _ptr(f), _ptr(A_log),
                                                   _ptr(dt_bias), _ptr(beta_logit), int(kind),
                                                   float(lower_bound), float(scale), float(eps),
                                                   _ptr(o))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_decode_step_gated failed ({rc})")
        return S, cs_out, o

    def layer_step(self, S, x, w, cs, f, A_log, dt_bias, beta_logit, scale, out_gate, norm_w,
                   kind=GATE_BOUNDED, lower_bound=-5.0, eps=L2NORM_EPS, norm_eps=RMSNORM_EPS):
        """decode_step_gated followed by the gated RMSNorm of every head:
        out_gate [M,H*D], norm_w [D].  Returns (S_new, cs_new, y [M,H,D])."""
        S = _f64(S).copy()
        M, H, D, _ = S.shape
        x, w, cs = _f64(x), _f64(w), _f64(cs)
        f, A_log, dt_bias, beta_logit = _f64(f), _f64(A_log), _f64(dt_bias), _f64(beta_logit)
        og, nw = _f64(out_gate), _f64(norm_w)
        assert og.shape == (M, H * D) and nw.shape == (D,)
        cs_out = np.empty_like(cs)
        y = np.empty((M, H, D))
        rc = self.lib.kda_oracle_layer_step(M, H, D, _ptr(S), _ptr(x), _ptr(w), _ptr(cs),
                                            _ptr(cs_out), _ptr(f), _ptr(A_log), _ptr(dt_bias),
                                            _ptr(beta_logit), int(kind), float(lower_bound),
                                            float(scale), float(eps), _ptr(og), _ptr(nw),
                                            float(norm_eps), _ptr(y))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_layer_step failed ({rc})")
        return S, cs_out, y


    def decode_multi(self, S, x, w, cs, alpha, beta, scale, eps=L2NORM_EPS):
        """T consecutive tokens per stream: x [M,T,3,H*D], alpha [M,T,H,D],
        beta [M,T,H]; S, w, cs as decode_step.  Returns (S_new, cs_new,
        o [M,T,H,D])."""
        S = _f64(S).copy()
        M, H, D, _ = S.shape
        x, w, cs = _f64(x), _f64(w), _f64(cs)
        alpha, beta = _f64(alpha), _f64(beta)
        T = x.shape[1]
        assert x.shape == (M, T, 3, H * D) and alpha.shape == (M, T, H, D) and beta.shape == (M, T, H)
        cs_out = np.empty_like(cs)
        o = np.empty((M, T, H, D))
        rc = self.lib.kda_oracle_decode_multi(T, M, H, D, _ptr(S), _ptr(x), _ptr(w), _ptr(cs),
                                              _ptr(cs_out), _ptr(alpha), _ptr(beta), float(scale),
                                              float(eps), _ptr(o))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_decode_multi failed ({rc})")
        return S, cs_out, o


    def sequence_gated(self, S, x, w, cs, f, A_log, dt_bias, beta_logit, scale,
                       kind=GATE_BOUNDED, lower_bound=-5.0, eps=L2NORM_EPS):
        """T tokens per stream with raw gate inputs: x [M,T,3,H*D], f [M,T,H*D],
        beta_logit [M,T,H]; A_log [H], dt_bias [H*D].  Returns (S_new, cs_new, o [M,T,H,D])."""
        S = _f64(S).copy()
        M, H, D, _ = S.shape
        x, w, cs = _f64(x), _f64(w), _f64(cs)
        f, A_log, dt_bias, beta_logit = _f64(f), _f64(A_log), _f64(dt_bias), _f64(beta_logit)
        T = x.shape[1]
        assert x.shape == (M, T, 3, H * D) and f.shape == (M, T, H * D) and beta_logit.shape == (M, T, H)
        cs_out = np.empty_like(cs)
        o = np.empty((M, T, H, D))
        rc = self.lib.kda_oracle_sequence_gated(T, M, H, D, _ptr(S), _ptr(x), _ptr(w), _ptr(cs), _ptr(cs_out),
                                                _ptr(f), _ptr(A_log), _ptr(dt_bias), _ptr(beta_logit),
                                                int(kind), float(lower_bound), float(scale), float(eps), _ptr(o))
        if rc != 0:
            raise RuntimeError(f"kda_oracle_sequence_gated failed ({rc})")
        return S, cs_out, o


_DEFAULT: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``kda_oracle.c`` (built on first use if missing)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
