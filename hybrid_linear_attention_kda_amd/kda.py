"""Python binding of ``libkda.so`` (argument marshalling only).

Each function has the name and argument order of its C entry point in
``include/kda.h``.  Shapes, dtypes and devices are derived from torch
tensors and checked here, because the C ABI receives bare pointers and
cannot see buffer sizes; every step of the computation runs in the HIP
kernels.  There is no fallback: if the library is not built, importing the
binding raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

#: the built library (see ``build.py``)
LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE = 0, 1, 2, 3
KDA_ERR_ALIGN, KDA_ERR_ALIAS, KDA_ERR_ARG, KDA_ERR_HIP = 4, 5, 6, 7
KDA_STATE_F32, KDA_STATE_BF16 = 0, 1
KDA_GATE_BOUNDED, KDA_GATE_SOFTPLUS = 0, 1

#: every symbol ``include/kda.h`` declares
EXPORTS = ("kda_decode_step", "kda_decode_step_split", "kda_decode_step_gated",
           "kda_decode_layer_step", "kda_decode_multi", "kda_prefill_gated", "kda_prefill_gated_ws",
           "kda_prefill_gated_noalloc", "kda_prefill_workspace_bytes", "kda_conv_step",
           "kda_recurrent_step", "kda_status_string", "kda_version")


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


_LIB = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the HIP library (once) and declare its C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built: run `python -m hybrid_linear_attention_kda_amd.build`")
    lib = ctypes.CDLL(path)
    i, f, vp, fp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p
    step = [i, i, i, i, vp, vp, vp, vp, vp, fp, fp, f, vp, vp]
    lib.kda_decode_step.argtypes = step
    lib.kda_decode_step.restype = i
    lib.kda_decode_step_split.argtypes = step + [i]
    lib.kda_decode_step_split.restype = i
    gated = [i, i, i, i, vp, vp, vp, vp, vp, vp, fp, fp, vp, i, f, f]
    lib.kda_decode_step_gated.argtypes = gated + [vp, vp]
    lib.kda_decode_step_gated.restype = i
    lib.kda_decode_layer_step.argtypes = gated + [vp, fp, f, vp, vp]
    lib.kda_decode_layer_step.restype = i
    lib.kda_decode_multi.argtypes = [i] + step
    lib.kda_decode_multi.restype = i
    lib.kda_prefill_gated.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, fp, fp, vp, f, f, vp, vp]
    lib.kda_prefill_gated.restype = i
    lib.kda_prefill_gated_ws.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, fp, fp, vp, f, f, vp, vp,
                                         ctypes.c_size_t, i, vp]
    lib.kda_prefill_gated_ws.restype = i
    lib.kda_prefill_gated_noalloc.argtypes = [i, i, i, i, i, vp, vp, vp, vp, vp, vp, fp, fp, vp, f, f, vp, vp]
    lib.kda_prefill_gated_noalloc.restype = i
    lib.kda_prefill_workspace_bytes.argtypes = [i, i, i, i]
    lib.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_conv_step.argtypes = [i, i, vp, vp, vp, vp, fp, vp]
    lib.kda_conv_step.restype = i
    lib.kda_recurrent_step.argtypes = [i, i, i, i, vp, fp, fp, fp, f, vp, vp]
    lib.kda_recurrent_step.restype = i
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = i
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load().kda_status_string(int(status)).decode()


def kda_status_string(status: int) -> str:
    return status_string(status)


def kda_version() -> int:
    return int(load().kda_version())


# ------------------------------------------------------------ marshalling --
def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device, stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _p(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _state_code(state: torch.Tensor) -> int:
    if state.dtype == torch.float32:
        return KDA_STATE_F32
    if state.dtype == torch.bfloat16:
        return KDA_STATE_BF16
    raise TypeError(f"state must be float32 or bfloat16, not {state.dtype}")


def _check(fn, rc):
    if rc != KDA_OK:
        raise KdaError(fn, rc)


def kda_decode_step(state, x_qkv, conv_w, conv_in, conv_out, alpha, beta, scale, o,
                    stream=None, nsplit: int | None = None):
    """Fused KDA decode step over M streams (see ``kda_decode_step`` in kda.h).

    state [M,H,D,D] f32|bf16 (in place), x_qkv [M,3,H*D] bf16,
    conv_w [3*H*D,4] bf16, conv_in/conv_out [M,3,3*H*D] bf16 (may be the same
    tensor), alpha [M,H,D] f32, beta [M,H] f32, o [M,H,D] bf16.
    ``nsplit`` forces the workgroups-per-head split (1, 2, 4).
    """
    lib = load()
    if state.dim() != 4:
        raise ValueError("state must be [M, H, D, D]")
    M, H, D, _ = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("state must be a GPU tensor")
    _need(state, "state", (M, H, D, D), state.dtype, dev)
    _need(x_qkv, "x_qkv", (M, 3, H * D), torch.bfloat16, dev)
    _need(conv_w, "conv_w", (3 * H * D, 4), torch.bfloat16, dev)
    _need(conv_in, "conv_in", (M, 3, 3 * H * D), torch.bfloat16, dev)
    _need(conv_out, "conv_out", (M, 3, 3 * H * D), torch.bfloat16, dev)
    _need(alpha, "alpha", (M, H, D), torch.float32, dev)
    _need(beta, "beta", (M, H), torch.float32, dev)
    _need(o, "o", (M, H, D), torch.bfloat16, dev)
    args = (M, H, D, _state_code(state), _p(state), _p(x_qkv), _p(conv_w), _p(conv_in),
            _p(conv_out), _p(alpha), _p(beta), float(scale), _p(o), _stream(dev, stream))
    if nsplit is None:
        _check("kda_decode_step", lib.kda_decode_step(*args))
    else:
        _check("kda_decode_step_split", lib.kda_decode_step_split(*args, int(nsplit)))


def kda_conv_step(x, conv_w, conv_in, conv_out, y, stream=None):
    """Conv + SiLU over C channels: x [M,C] bf16, conv_w [C,4] bf16,
    conv_in/conv_out [M,3,C] bf16, y [M,C] f32."""
    lib = load()
    if x.dim() != 2:
        raise ValueError("x must be [M, C]")
    M, C = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    _need(x, "x", (M, C), torch.bfloat16, dev)
    _need(conv_w, "conv_w", (C, 4), torch.bfloat16, dev)
    _need(conv_in, "conv_in", (M, 3, C), torch.bfloat16, dev)
    _need(conv_out, "conv_out", (M, 3, C), torch.bfloat16, dev)
    _need(y, "y", (M, C), torch.float32, dev)
    _check("kda_conv_step", lib.kda_conv_step(M, C, _p(x), _p(conv_w), _p(conv_in), _p(conv_out),
                                              _p(y), _stream(dev, stream)))


def kda_recurrent_step(state, qkv, alpha, beta, scale, o, stream=None):
    """Recurrent part from post-conv q|k|v [M,3,H*D] f32; other args as kda_decode_step."""
    lib = load()
    if state.dim() != 4:
        raise ValueError("state must be [M, H, D, D]")
    M, H, D, _ = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("state must be a GPU tensor")
    _need(state, "state", (M, H, D, D), state.dtype, dev)
    _need(qkv, "qkv", (M, 3, H * D), torch.float32, dev)
    _need(alpha, "alpha", (M, H, D), torch.float32, dev)
    _need(beta, "beta", (M, H), torch.float32, dev)
    _need(o, "o", (M, H, D), torch.bfloat16, dev)
    _check("kda_recurrent_step",
           lib.kda_recurrent_step(M, H, D, _state_code(state), _p(state), _p(qkv), _p(alpha),
                                  _p(beta), float(scale), _p(o), _stream(dev, stream)))


def _gated_args(state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log, dt_bias, beta_logit,
                gate_kind, lower_bound, scale):
    if state.dim() != 4:
        raise ValueError("state must be [M, H, D, D]")
    M, H, D, _ = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("state must be a GPU tensor")
    _need(state, "state", (M, H, D, D), state.dtype, dev)
    _need(x_qkv, "x_qkv", (M, 3, H * D), torch.bfloat16, dev)
    _need(conv_w, "conv_w", (3 * H * D, 4), torch.bfloat16, dev)
    _need(conv_in, "conv_in", (M, 3, 3 * H * D), torch.bfloat16, dev)
    _need(conv_out, "conv_out", (M, 3, 3 * H * D), torch.bfloat16, dev)
    _need(f_gate, "f_gate", (M, H * D), torch.bfloat16, dev)
    _need(A_log, "A_log", (H,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * D,), torch.float32, dev)
    _need(beta_logit, "beta_logit", (M, H), torch.bfloat16, dev)
    return (M, H, D, dev), (M, H, D, _state_code(state), _p(state), _p(x_qkv), _p(conv_w),
                            _p(conv_in), _p(conv_out), _p(f_gate), _p(A_log), _p(dt_bias),
                            _p(beta_logit), int(gate_kind), float(lower_bound), float(scale))


def kda_decode_step_gated(state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log, dt_bias,
                          beta_logit, scale, o, gate_kind=KDA_GATE_BOUNDED, lower_bound=-5.0,
                          stream=None):
    """Fused step with raw gate inputs (see ``kda_decode_step_gated`` in kda.h):
    f_gate [M,H*D] bf16, A_log [H] f32, dt_bias [H*D] f32, beta_logit [M,H]
    bf16; o [M,H,D] bf16; the rest as kda_decode_step."""
    lib = load()
    (M, H, D, dev), args = _gated_args(state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log,
                                       dt_bias, beta_logit, gate_kind, lower_bound, scale)
    _need(o, "o", (M, H, D), torch.bfloat16, dev)
    _check("kda_decode_step_gated", lib.kda_decode_step_gated(*args, _p(o), _stream(dev, stream)))


def kda_decode_layer_step(state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log, dt_bias,
                          beta_logit, scale, out_gate, norm_weight, y,
                          gate_kind=KDA_GATE_BOUNDED, lower_bound=-5.0, norm_eps=1e-5,
                          stream=None):
    """The gated step followed by the gated RMSNorm of every head (see
    ``kda_decode_layer_step`` in kda.h): out_gate [M,H*D] bf16, norm_weight
    [D] f32, y [M,H,D] bf16."""
    lib = load()
    (M, H, D, dev), args = _gated_args(state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log,
                                       dt_bias, beta_logit, gate_kind, lower_bound, scale)
    _need(out_gate, "out_gate", (M, H * D), torch.bfloat16, dev)
    _need(norm_weight, "norm_weight", (D,), torch.float32, dev)
    _need(y, "y", (M, H, D), torch.bfloat16, dev)
    _check("kda_decode_layer_step",
           lib.kda_decode_layer_step(*args, _p(out_gate), _p(norm_weight), float(norm_eps), _p(y),
                                     _stream(dev, stream)))


def kda_decode_multi(state, x_qkv, conv_w, conv_in, conv_out, alpha, beta, scale, o, stream=None):
    """T tokens per stream in one call (see ``kda_decode_multi`` in kda.h):
    x_qkv [M,T,3,H*D] bf16, alpha [M,T,H,D] f32, beta [M,T,H] f32,
    o [M,T,H,D] bf16; state, conv_w, conv_in/conv_out as kda_decode_step."""
    lib = load()
    if state.dim() != 4 or x_qkv.dim() != 4:
        raise ValueError("state must be [M, H, D, D] and x_qkv [M, T, 3, H*D]")
    M, H, D, _ = state.shape
    T = x_qkv.shape[1]
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("state must be a GPU tensor")
    _need(state, "state", (M, H, D, D), state.dtype, dev)
    _need(x_qkv, "x_qkv", (M, T, 3, H * D), torch.bfloat16, dev)
    _need(conv_w, "conv_w", (3 * H * D, 4), torch.bfloat16, dev)
    _need(conv_in, "conv_in", (M, 3, 3 * H * D), torch.bfloat16, dev)
    _need(conv_out, "conv_out", (M, 3, 3 * H * D), torch.bfloat16, dev)
    _need(alpha, "alpha", (M, T, H, D), torch.float32, dev)
    _need(beta, "beta", (M, T, H), torch.float32, dev)
    _need(o, "o", (M, T, H, D), torch.bfloat16, dev)
    _check("kda_decode_multi",
           lib.kda_decode_multi(T, M, H, D, _state_code(state), _p(state), _p(x_qkv), _p(conv_w),
                                _p(conv_in), _p(conv_out), _p(alpha), _p(beta), float(scale), _p(o),
                                _stream(dev, stream)))


def kda_prefill_workspace_bytes(L: int, M: int, H: int, D: int) -> int:
    """Workspace for a one-segment kda_prefill_gated_ws call (0: invalid shape)."""
    return int(load().kda_prefill_workspace_bytes(int(L), int(M), int(H), int(D)))


def kda_prefill_gated(state, x_qkv, conv_w, conv_in, conv_out, f_gate, A_log, dt_bias, beta_logit,
                      scale, o, lower_bound=-5.0, stream=None, workspace=None, passes=0):
    """L tokens per stream, chunkwise on matrix cores (see ``kda_prefill_gated``
    in kda.h): x_qkv [M,L,3,H*D] bf16, f_gate [M,L,H*D] bf16, A_log [H] f32,
    dt_bias [H*D] f32, beta_logit [M,L,H] bf16, o [M,L,H,D] bf16; D = 128.
    With ``workspace`` (a contiguous GPU tensor of any dtype) the call goes to
    ``kda_prefill_gated_ws`` with ``passes`` (0 choose, 1 one pass, 2 two
    passes); with ``workspace="noalloc"`` to ``kda_prefill_gated_noalloc``."""
    lib = load()
    if state.dim() != 4 or x_qkv.dim() != 4:
        raise ValueError("state must be [M, H, D, D] and x_qkv [M, L, 3, H*D]")
    M, H, D, _ = state.shape
    L = x_qkv.shape[1]
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("state must be a GPU tensor")
    _need(state, "state", (M, H, D, D), state.dtype, dev)
    _need(x_qkv, "x_qkv", (M, L, 3, H * D), torch.bfloat16, dev)
    _need(conv_w, "conv_w", (3 * H * D, 4), torch.bfloat16, dev)
    _need(conv_in, "conv_in", (M, 3, 3 * H * D), torch.bfloat16, dev)
    _need(conv_out, "conv_out", (M, 3, 3 * H * D), torch.bfloat16, dev)
    _need(f_gate, "f_gate", (M, L, H * D), torch.bfloat16, dev)
    _need(A_log, "A_log", (H,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * D,), torch.float32, dev)
    _need(beta_logit, "beta_logit", (M, L, H), torch.bfloat16, dev)
    _need(o, "o", (M, L, H, D), torch.bfloat16, dev)
    if workspace is None:
        _check("kda_prefill_gated",
               lib.kda_prefill_gated(L, M, H, D, _state_code(state), _p(state), _p(x_qkv), _p(conv_w),
                                     _p(conv_in), _p(conv_out), _p(f_gate), _p(A_log), _p(dt_bias),
                                     _p(beta_logit), float(lower_bound), float(scale), _p(o),
                                     _stream(dev, stream)))
        return
    if isinstance(workspace, str):
        if workspace != "noalloc":
            raise ValueError("workspace must be a tensor or 'noalloc'")
        _check("kda_prefill_gated_noalloc",
               lib.kda_prefill_gated_noalloc(L, M, H, D, _state_code(state), _p(state), _p(x_qkv), _p(conv_w),
                                             _p(conv_in), _p(conv_out), _p(f_gate), _p(A_log), _p(dt_bias),
                                             _p(beta_logit), float(lower_bound), float(scale), _p(o),
                                             _stream(dev, stream)))
        return
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the state's device")
    _check("kda_prefill_gated_ws",
           lib.kda_prefill_gated_ws(L, M, H, D, _state_code(state), _p(state), _p(x_qkv), _p(conv_w),
                                    _p(conv_in), _p(conv_out), _p(f_gate), _p(A_log), _p(dt_bias),
                                    _p(beta_logit), float(lower_bound), float(scale), _p(o), _p(workspace),
                                    workspace.numel() * workspace.element_size(), int(passes),
                                    _stream(dev, stream)))
