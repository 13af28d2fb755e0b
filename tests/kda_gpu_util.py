"""Helpers shared by the GPU parity tests: device buffers for one layer,
the per-(stream, head) sub-problem the oracle can evaluate one by one, and
the error metric of the pages (max |gpu - ref| over max |ref|)."""
from __future__ import annotations

import numpy as np
import torch

import kda_synth
from hybrid_linear_attention_kda_amd import kda_decode_step

# tolerances of the decode step, relative to the largest reference magnitude
TOL_STATE_F32 = 1e-5
TOL_STATE_BF16 = 4e-3
TOL_O = 4e-3


def tol_state(state_dtype: str) -> float:
    return TOL_STATE_F32 if state_dtype == "f32" else TOL_STATE_BF16


def rel_err(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    den = float(np.max(np.abs(r)))
    err = float(np.max(np.abs(g - r)))
    return err / den if den > 0 else err


def host(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (bf16/f32 widen exactly)."""
    return t.detach().to(torch.float64).cpu().numpy()


class Layer:
    """Device buffers of one layer: state, conv weights, conv state, output."""

    def __init__(self, wl, layer, device, state_dtype="f32", inplace=True):
        li = kda_synth.layer_inputs(wl, layer, device, state_dtype)
        self.wl, self.layer, self.state_dtype = wl, layer, state_dtype
        self.state = li["state"]
        self.conv_w = li["conv_w"]
        self.conv = li["conv_state"]
        self.conv_alt = None if inplace else torch.empty_like(self.conv)
        self.o = torch.empty((wl.M, wl.H, wl.D), dtype=torch.bfloat16, device=device)

    def step(self, inp, nsplit=None, stream=None):
        cin = self.conv
        cout = self.conv if self.conv_alt is None else self.conv_alt
        kda_decode_step(self.state, inp["x"], self.conv_w, cin, cout, inp["alpha"], inp["beta"],
                        self.wl.scale, self.o, stream=stream, nsplit=nsplit)
        if self.conv_alt is not None:
            self.conv, self.conv_alt = self.conv_alt, self.conv


# --------------------------------------------------- one (stream, head) unit --
def unit_inputs(wl, m, h, conv_w, conv, inp=None):
    """Slice the inputs of stream m, head h into an H = 1 problem (float64).

    Channel c of tensor t (q, k, v) of head h lives at t*H*D + h*D + c; the
    conv is depthwise, so a head's channels form a problem of their own."""
    H, D = wl.H, wl.D
    out = {
        "conv_w": host(conv_w).reshape(3, H, D, 4)[:, h].reshape(3 * D, 4),
        "conv": host(conv[m]).reshape(3, 3, H, D)[:, :, h].reshape(1, 3, 3 * D),
    }
    if inp is not None:
        out["x"] = host(inp["x"][m]).reshape(3, H, D)[:, h].reshape(1, 3, D)
        out["alpha"] = host(inp["alpha"][m, h]).reshape(1, 1, D)
        out["beta"] = host(inp["beta"][m, h]).reshape(1, 1)
    return out


def step_unit_inputs(wl, m, h, inp):
    H, D = wl.H, wl.D
    return {
        "x": host(inp["x"][m]).reshape(3, H, D)[:, h].reshape(1, 3, D),
        "alpha": host(inp["alpha"][m, h]).reshape(1, 1, D),
        "beta": host(inp["beta"][m, h]).reshape(1, 1),
    }
