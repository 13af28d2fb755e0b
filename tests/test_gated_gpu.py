"""GPU parity of the gated step and the layer step (through the C ABI)
against the CPU oracle.

kda_decode_step_gated forms alpha from the raw forget gate and beta from its
logit inside the kernel ("GLM-5.3 deep dive" 8.2.3, 8.2.4 steps 4-5);
kda_decode_layer_step adds the gated RMSNorm of each head's outputs (8.2.4
step 7).  The oracle evaluates the same definitions in double.  Tolerances
(relative to the largest reference magnitude, as for the plain step):
state 1e-5 (f32) / 4e-3 (bf16), o and y 4e-3 (one bf16 rounding).
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from hybrid_linear_attention_kda_amd import (KDA_GATE_BOUNDED, KDA_GATE_SOFTPLUS,
                                             kda_decode_layer_step, kda_decode_step_gated)
from kda_gpu_util import TOL_O, host, rel_err, tol_state

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def say(msg):
    print(msg, flush=True)


class GatedLayer:
    """Device buffers of one layer for the gated entry points."""

    def __init__(self, wl, layer, state_dtype, inplace=True):
        li = kda_synth.layer_inputs(wl, layer, DEV, state_dtype)
        gp = kda_synth.gate_params(wl, layer, DEV)
        self.wl, self.layer, self.state_dtype = wl, layer, state_dtype
        self.state, self.conv_w, self.conv = li["state"], li["conv_w"], li["conv_state"]
        self.A_log, self.dt_bias, self.norm_w = gp["A_log"], gp["dt_bias"], gp["norm_w"]
        self.conv_alt = None if inplace else torch.empty_like(self.conv)
        self.out = torch.empty((wl.M, wl.H, wl.D), dtype=torch.bfloat16, device=DEV)

    def step(self, inp, gi, kind, lb, layer_step):
        cin = self.conv
        cout = self.conv if self.conv_alt is None else self.conv_alt
        if layer_step:
            kda_decode_layer_step(self.state, inp["x"], self.conv_w, cin, cout, gi["f"], self.A_log,
                                  self.dt_bias, gi["beta_logit"], self.wl.scale, gi["out_gate"],
                                  self.norm_w, self.out, gate_kind=kind, lower_bound=lb)
        else:
            kda_decode_step_gated(self.state, inp["x"], self.conv_w, cin, cout, gi["f"], self.A_log,
                                  self.dt_bias, gi["beta_logit"], self.wl.scale, self.out,
                                  gate_kind=kind, lower_bound=lb)
        if self.conv_alt is not None:
            self.conv, self.conv_alt = self.conv_alt, self.conv


def check_step(orc, lay, S_ref, cs_ref, t, kind, lb, layer_step, teacher):
    """One GPU step and the oracle's; returns (S_ref, cs_ref, (e_out, e_state))."""
    wl = lay.wl
    inp = kda_synth.step_inputs(wl, lay.layer, t, DEV)
    gi = kda_synth.gate_inputs(wl, lay.layer, t, DEV)
    S_in = host(lay.state) if teacher else S_ref
    lay.step(inp, gi, kind, lb, layer_step)
    torch.cuda.synchronize()
    args = (S_in, host(inp["x"]), host(lay.conv_w), cs_ref, host(gi["f"]), host(lay.A_log),
            host(lay.dt_bias), host(gi["beta_logit"]), wl.scale)
    if layer_step:
        S_ref, cs_ref, out_ref = orc.layer_step(*args, host(gi["out_gate"]), host(lay.norm_w),
                                                kind=kind, lower_bound=lb)
    else:
        S_ref, cs_ref, out_ref = orc.decode_step_gated(*args, kind=kind, lower_bound=lb)
    e_o = rel_err(host(lay.out), out_ref)
    e_s = rel_err(host(lay.state), S_ref)
    assert np.array_equal(host(lay.conv), cs_ref), "conv state must advance bit-exactly"
    assert e_o <= TOL_O, f"output error {e_o:.3e}"
    assert e_s <= tol_state(lay.state_dtype), f"state error {e_s:.3e}"
    return S_ref, cs_ref, (e_o, e_s)


KINDS = [(KDA_GATE_BOUNDED, -5.0), (KDA_GATE_SOFTPLUS, 0.0)]


@pytest.mark.parametrize("layer_step", [False, True], ids=["gated", "layer"])
@pytest.mark.parametrize("kind,lb", KINDS, ids=["bounded", "softplus"])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,H,D", [(1, 4, 16), (2, 3, 32), (3, 2, 64), (3, 5, 128), (2, 64, 128), (8, 64, 128)])
def test_gated_against_oracle(orc, M, H, D, state_dtype, kind, lb, layer_step):
    """Three consecutive steps; f32 state free-running, bf16 teacher-forced."""
    wl = kda_synth.custom(f"gated_{M}_{H}_{D}", M, H, D, steps=3)
    lay = GatedLayer(wl, 0, state_dtype)
    S_ref, cs_ref = host(lay.state), host(lay.conv)
    worst = [0.0, 0.0]
    for t in range(wl.steps):
        S_ref, cs_ref, e = check_step(orc, lay, S_ref, cs_ref, t, kind, lb, layer_step,
                                      teacher=state_dtype == "bf16")
        worst = [max(a, b) for a, b in zip(worst, e)]
    say(f"{'layer' if layer_step else 'gated'} {kind} {state_dtype} ({M},{H},{D}): "
        f"out {worst[0]:.3e} state {worst[1]:.3e}")


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_gated_split_path(orc, state_dtype):
    """M*H below the CU count with distinct conv buffers: the library splits
    each head's columns over workgroups; every split forms the full alpha."""
    wl = kda_synth.custom("gated_split", 1, 64, 128, steps=2)
    lay = GatedLayer(wl, 0, state_dtype, inplace=False)
    S_ref, cs_ref = host(lay.state), host(lay.conv)
    for t in range(wl.steps):
        S_ref, cs_ref, e = check_step(orc, lay, S_ref, cs_ref, t, KDA_GATE_BOUNDED, -5.0, False,
                                      teacher=state_dtype == "bf16")
    say(f"gated split {state_dtype}: out {e[0]:.3e} state {e[1]:.3e}")


@pytest.mark.parametrize("layer_step", [False, True], ids=["gated", "layer"])
@pytest.mark.parametrize("state_dtype,M,H", [("f32", 33, 64), ("bf16", 33, 64), ("f32", 33, 63)])
def test_gated_wide_grid(orc, state_dtype, layer_step, M, H):
    """33 x 64 = 2112 heads, whole tensors: the launches that store the state
    with agent scope (from 2048 heads on), with a partial last round of
    workgroups.  For an f32 state also 33 x 63 = 2079 heads: the 16-wave
    grid alternates between the two halves of the heads only when their
    number is even, and runs them in order otherwise."""
    wl = kda_synth.custom("gated_wide", M, H, 128, steps=2)
    lay = GatedLayer(wl, 0, state_dtype)
    S_ref, cs_ref = host(lay.state), host(lay.conv)
    for t in range(wl.steps):
        S_ref, cs_ref, e = check_step(orc, lay, S_ref, cs_ref, t, KDA_GATE_BOUNDED, -5.0, layer_step,
                                      teacher=state_dtype == "bf16")
    say(f"{'layer' if layer_step else 'gated'} wide {M}x{H} {state_dtype}: out {e[0]:.3e} state {e[1]:.3e}")


def test_layer_step_glm_m32_sampled(orc):
    """Full geometry, M = 32 (the launch shape the benchmark times): the
    whole layer against the oracle on sampled (stream, head) units."""
    wl = kda_synth.Workload(**{**kda_synth.WORKLOADS["glm_m32"].__dict__, "layers": 1, "steps": 2})
    lay = GatedLayer(wl, 0, "f32")
    H, D = wl.H, wl.D
    units = [(0, 0), (7, 13), (31, 63), (16, 40)]
    refs = {}
    for (m, h) in units:
        refs[(m, h)] = (host(lay.state[m, h])[None, None], host(lay.conv[m]).reshape(3, 3, H, D)[:, :, h]
                        .reshape(1, 3, 3 * D))
    cw = host(lay.conv_w).reshape(3, H, D, 4)
    for t in range(wl.steps):
        inp = kda_synth.step_inputs(wl, 0, t, DEV)
        gi = kda_synth.gate_inputs(wl, 0, t, DEV)
        lay.step(inp, gi, KDA_GATE_BOUNDED, -5.0, True)
        torch.cuda.synchronize()
        for (m, h) in units:
            S_ref, cs_ref = refs[(m, h)]
            sl = slice(h * D, (h + 1) * D)
            S_ref, cs_ref, y_ref = orc.layer_step(
                S_ref, host(inp["x"][m]).reshape(3, H, D)[:, h].reshape(1, 3, D),
                cw[:, h].reshape(3 * D, 4), cs_ref, host(gi["f"][m, sl])[None],
                host(lay.A_log[h:h + 1]), host(lay.dt_bias[sl]), host(gi["beta_logit"][m, h:h + 1])[None],
                wl.scale, host(gi["out_gate"][m, sl])[None], host(lay.norm_w))
            refs[(m, h)] = (S_ref, cs_ref)
            assert rel_err(host(lay.state[m, h]), S_ref[0, 0]) <= 1e-5, f"state ({m},{h}) step {t}"
            assert rel_err(host(lay.out[m, h]), y_ref[0, 0]) <= TOL_O, f"y ({m},{h}) step {t}"
    say("layer step glm_m32 sampled units ok")


def test_gated_equals_plain_step_with_host_gate(orc):
    """The gated kernel against the plain kernel fed with alpha and beta that
    the oracle formed from the same raw inputs (rounded to f32): the two GPU
    paths agree to f32 rounding of the gate."""
    from kda_gpu_util import Layer
    wl = kda_synth.custom("gated_vs_plain", 4, 8, 128, steps=1)
    g = GatedLayer(wl, 0, "f32")
    p = Layer(wl, 0, DEV, "f32")
    inp = kda_synth.step_inputs(wl, 0, 0, DEV)
    gi = kda_synth.gate_inputs(wl, 0, 0, DEV)
    f, A, b = host(gi["f"]), host(g.A_log), host(g.dt_bias)
    alpha = np.stack([np.stack([orc.gate(f[m, h * 128:(h + 1) * 128], A[h], b[h * 128:(h + 1) * 128])
                                for h in range(wl.H)]) for m in range(wl.M)])
    beta = orc.beta(host(gi["beta_logit"]))
    inp2 = dict(inp, alpha=torch.tensor(alpha, dtype=torch.float32, device=DEV),
                beta=torch.tensor(beta, dtype=torch.float32, device=DEV))
    g.step(inp, gi, KDA_GATE_BOUNDED, -5.0, False)
    p.step(inp2)
    torch.cuda.synchronize()
    assert torch.equal(g.conv, p.conv)
    assert rel_err(host(g.state), host(p.state)) <= 2e-6
    assert rel_err(host(g.out), host(p.o)) <= 2 ** -7
