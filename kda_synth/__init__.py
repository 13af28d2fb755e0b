"""Seeded synthetic inputs for the KDA decode step.

This module only draws random numbers and shapes them; it holds none of the
decode step's arithmetic.  Both the GPU library's tests/benchmark and the CPU
oracle take their inputs from here.

Every tensor is drawn from its own ``torch.Generator`` seeded by
``seed_for(workload, layer, step, what)``, on the device the caller names.  A
given (workload, device type) always yields the same values; CPU and GPU
generators are different streams, so a GPU parity test draws on the GPU and
hands the oracle a host copy of the very same tensors.

Distributions (the workloads the pages measure use synthetic random inputs at
the real dims; "N(0, s)" below means standard deviation s):

* initial state ~ N(0, 0.1), rounded to BF16 (round-to-nearest-even) so that
  FP32 and BF16 storage start from identical values;
* pre-conv q|k|v ~ N(0, 1) and conv weights ~ N(0, 0.5), both BF16;
* conv state: zeros for the tiny workload, else N(0, 1) in BF16 (the raw
  inputs of three earlier tokens);
* alpha: tiny workload exp(-softplus(g)), g ~ N(0, 1), evaluated in double
  and rounded once to FP32; the full-size workloads 0.9 + 0.1 U(0, 1), and the
  serving-scale workload U(0.5, 1);
* beta: sigmoid(N(0, 1)) per head in double, rounded to FP32; the
  serving-scale workload U(0, 1) with heads 0..4 of every stream pinned to
  0, 2^-24, 0.5, 1 - 2^-24 and 1.

Raw gate inputs for the gated step and the layer step (trained values are
not available; these put the keep factor mostly in (0.6, 0.99)):

* A_log ~ U(-0.5, 0.5) per head and dt_bias ~ N(-4, 1) per channel, FP32,
  fixed per layer;
* forget-gate projection f ~ N(0, 1), BF16, per token;
* write-strength logits ~ N(0, 1), BF16, per token;
* output gate ~ N(0, 1), BF16, per token; RMSNorm weight 1 + 0.1 N(0, 1),
  FP32, fixed per layer.

Whole sequences for the chunked prefill (``sequence_inputs``) draw the same
distributions once per tensor for all L tokens (one generator each), so a
long prompt costs one draw instead of L.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import torch

BF16 = torch.bfloat16
F32 = torch.float32


@dataclass(frozen=True)
class Workload:
    name: str
    M: int          # streams
    H: int          # heads
    D: int          # dk = dv
    layers: int     # layers with distinct states
    steps: int      # consecutive decode steps
    state_dtypes: tuple
    alpha_kind: str  # "gate", "u09", "u05"
    beta_kind: str   # "sigmoid", "uniform_tails"
    conv_init: str   # "zero", "normal"
    seed: int = 0
    description: str = ""

    @property
    def scale(self) -> float:
        """q scale 1/sqrt(D), rounded to FP32."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=F32).item())

    def state_bytes(self, state_dtype: str) -> int:
        """Bytes of recurrent state per layer (all streams)."""
        return self.M * self.H * self.D * self.D * (4 if state_dtype == "f32" else 2)


WORKLOADS = {
    "tiny": Workload("tiny", M=1, H=4, D=16, layers=1, steps=16, state_dtypes=("f32", "bf16"),
                     alpha_kind="gate", beta_kind="sigmoid", conv_init="zero", seed=0,
                     description="1 stream, 1 layer, 4 heads, dk=dv=16, 16 sequential steps"),
    "glm_m1": Workload("glm_m1", M=1, H=64, D=128, layers=1, steps=1, state_dtypes=("f32", "bf16"),
                       alpha_kind="u09", beta_kind="sigmoid", conv_init="normal", seed=1,
                       description="GLM-5.3-Flash KDA layer, 64x128x128, one step, M=1"),
    "glm_m8": Workload("glm_m8", M=8, H=64, D=128, layers=34, steps=1, state_dtypes=("f32", "bf16"),
                       alpha_kind="u09", beta_kind="sigmoid", conv_init="normal", seed=2,
                       description="M=8 streams, 34 layers with distinct states, one step"),
    "glm_m32": Workload("glm_m32", M=32, H=64, D=128, layers=34, steps=8, state_dtypes=("f32", "bf16"),
                        alpha_kind="u09", beta_kind="sigmoid", conv_init="normal", seed=3,
                        description="M=32 streams, 34 layers, FP32 state, 8 consecutive steps"),
    "glm_m128": Workload("glm_m128", M=128, H=64, D=128, layers=34, steps=8, state_dtypes=("bf16",),
                         alpha_kind="u05", beta_kind="uniform_tails", conv_init="normal", seed=4,
                         description="M=128 streams, 34 layers, BF16 state, 8 steps, beta tails"),
}

#: beta values pinned on heads 0..4 of the serving-scale workload.
BETA_TAILS = (0.0, 2.0 ** -24, 0.5, 1.0 - 2.0 ** -24, 1.0)


def seed_for(wl: Workload, layer: int, step: int, what: str) -> int:
    key = f"{wl.name}/{wl.seed}/{layer}/{step}/{what}".encode()
    return int.from_bytes(hashlib.sha256(key).digest()[:8], "little") & ((1 << 63) - 1)


def _gen(wl, layer, step, what, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(wl, layer, step, what))
    return g


def _randn(shape, g, device, dtype=F32):
    return torch.randn(shape, generator=g, device=device, dtype=dtype)


def initial_state(wl: Workload, layer: int, device, state_dtype: str = "f32") -> torch.Tensor:
    """[M, H, D, D] initial recurrent state, N(0, 0.1) rounded to BF16."""
    g = _gen(wl, layer, 0, "state", device)
    s = (_randn((wl.M, wl.H, wl.D, wl.D), g, device) * 0.1).to(BF16)
    return s if state_dtype == "bf16" else s.to(F32)


def conv_weights(wl: Workload, layer: int, device) -> torch.Tensor:
    """[3*H*D, 4] BF16 depthwise conv weights (q channels, then k, then v)."""
    g = _gen(wl, layer, 0, "conv_w", device)
    return (_randn((3 * wl.H * wl.D, 4), g, device) * 0.5).to(BF16)


def conv_state(wl: Workload, layer: int, device) -> torch.Tensor:
    """[M, 3, 3*H*D] BF16 conv state, tap 0 oldest."""
    shape = (wl.M, 3, 3 * wl.H * wl.D)
    if wl.conv_init == "zero":
        return torch.zeros(shape, dtype=BF16, device=device)
    g = _gen(wl, layer, 0, "conv_state", device)
    return _randn(shape, g, device).to(BF16)


def step_inputs(wl: Workload, layer: int, step: int, device) -> dict:
    """Per-token inputs: x [M,3,H*D] BF16, alpha [M,H,D] FP32, beta [M,H] FP32."""
    M, H, D = wl.M, wl.H, wl.D
    x = _randn((M, 3, H * D), _gen(wl, layer, step, "x", device), device).to(BF16)
    ga = _gen(wl, layer, step, "alpha", device)
    if wl.alpha_kind == "gate":
        graw = _randn((M, H, D), ga, device, torch.float64)
        alpha = (1.0 / (1.0 + torch.exp(graw))).to(F32)      # exp(-softplus(g))
    elif wl.alpha_kind == "u09":
        alpha = (0.9 + 0.1 * torch.rand((M, H, D), generator=ga, device=device,
                                        dtype=torch.float64)).to(F32)
    elif wl.alpha_kind == "u05":
        alpha = (0.5 + 0.5 * torch.rand((M, H, D), generator=ga, device=device,
                                        dtype=torch.float64)).to(F32)
    else:
        raise ValueError(wl.alpha_kind)
    gb = _gen(wl, layer, step, "beta", device)
    if wl.beta_kind == "sigmoid":
        beta = torch.sigmoid(_randn((M, H), gb, device, torch.float64)).to(F32)
    elif wl.beta_kind == "uniform_tails":
        beta = torch.rand((M, H), generator=gb, device=device, dtype=torch.float64)
        for i, val in enumerate(BETA_TAILS[:H]):
            beta[:, i] = val
        beta = beta.to(F32)
    else:
        raise ValueError(wl.beta_kind)
    return {"x": x, "alpha": alpha, "beta": beta}


def layer_inputs(wl: Workload, layer: int, device, state_dtype: str = "f32") -> dict:
    """Everything one layer needs before its first step."""
    return {
        "state": initial_state(wl, layer, device, state_dtype),
        "conv_w": conv_weights(wl, layer, device),
        "conv_state": conv_state(wl, layer, device),
    }


def custom(name: str, M: int, H: int, D: int, *, steps: int = 1, layers: int = 1,
           alpha_kind: str = "u09", beta_kind: str = "sigmoid", conv_init: str = "normal",
           seed: int = 100) -> Workload:
    """An ad-hoc workload for edge-case tests (ragged M/H, other D)."""
    return Workload(name, M=M, H=H, D=D, layers=layers, steps=steps,
                    state_dtypes=("f32", "bf16"), alpha_kind=alpha_kind,
                    beta_kind=beta_kind, conv_init=conv_init, seed=seed)


def gate_params(wl: Workload, layer: int, device) -> dict:
    """Per-layer gate and norm parameters: A_log [H], dt_bias [H*D], norm_w [D] (FP32)."""
    H, D = wl.H, wl.D
    ga = _gen(wl, layer, 0, "A_log", device)
    A_log = (torch.rand((H,), generator=ga, device=device, dtype=torch.float64) - 0.5).to(F32)
    dt_bias = (_randn((H * D,), _gen(wl, layer, 0, "dt_bias", device), device) - 4.0).to(F32)
    norm_w = (1.0 + 0.1 * _randn((D,), _gen(wl, layer, 0, "norm_w", device), device)).to(F32)
    return {"A_log": A_log, "dt_bias": dt_bias, "norm_w": norm_w}


def gate_inputs(wl: Workload, layer: int, step: int, device) -> dict:
    """Per-token raw gate inputs: f [M,H*D], beta_logit [M,H], out_gate [M,H*D], all BF16."""
    M, H, D = wl.M, wl.H, wl.D
    f = _randn((M, H * D), _gen(wl, layer, step, "f_gate", device), device).to(BF16)
    bl = _randn((M, H), _gen(wl, layer, step, "beta_logit", device), device).to(BF16)
    og = _randn((M, H * D), _gen(wl, layer, step, "out_gate", device), device).to(BF16)
    return {"f": f, "beta_logit": bl, "out_gate": og}


def sequence_inputs(wl: Workload, layer: int, L: int, device) -> dict:
    """L tokens at once for the chunked prefill: x [M,L,3,H*D], f [M,L,H*D],
    beta_logit [M,L,H], all BF16, the per-token distributions."""
    M, H, D = wl.M, wl.H, wl.D
    x = _randn((M, L, 3, H * D), _gen(wl, layer, -1, "seq_x", device), device).to(BF16)
    f = _randn((M, L, H * D), _gen(wl, layer, -1, "seq_f_gate", device), device).to(BF16)
    bl = _randn((M, L, H), _gen(wl, layer, -1, "seq_beta_logit", device), device).to(BF16)
    return {"x": x, "f": f, "beta_logit": bl}
