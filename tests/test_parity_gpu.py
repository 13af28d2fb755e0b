"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Inputs are drawn on the GPU by ``kda_synth`` and handed to the oracle as
exact float64 host copies.  Tolerances, relative to the largest reference
magnitude: state 1e-5 (f32 storage) / 4e-3 (bf16 storage), output 4e-3.
Multi-step f32 runs are compared free-running; multi-step bf16 runs are
compared with teacher forcing (the oracle restarts each step from the
GPU's stored state, which is exact in double), so each check sees exactly
one bf16 rounding.
"""
import math

import numpy as np
import pytest
import torch

import kda_synth
import oracle
from kda_gpu_util import (TOL_O, Layer, host, rel_err, step_unit_inputs, tol_state,
                          unit_inputs)

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


def full_step_check(orc, lay, S_ref, cs_ref, inp, tol_s, teacher=False):
    """Run one GPU step and the oracle step; return (S_ref, cs_ref, errs)."""
    wl = lay.wl
    S_in = host(lay.state) if teacher else S_ref
    lay.step(inp)
    torch.cuda.synchronize()
    S_ref, cs_ref, o_ref = orc.decode_step(S_in, host(inp["x"]), host(lay.conv_w), cs_ref,
                                           host(inp["alpha"]), host(inp["beta"]), wl.scale)
    e_o = rel_err(host(lay.o), o_ref)
    e_s = rel_err(host(lay.state), S_ref)
    assert np.array_equal(host(lay.conv), cs_ref), "conv state must advance bit-exactly"
    assert e_o <= TOL_O, f"output error {e_o:.3e}"
    assert e_s <= tol_s, f"state error {e_s:.3e}"
    return S_ref, cs_ref, (e_o, e_s)


# ----------------------------------------------------------------- tiny ----
def test_tiny_f32_free_running(orc):
    wl = kda_synth.WORKLOADS["tiny"]
    lay = Layer(wl, 0, DEV, "f32")
    S_ref, cs_ref = host(lay.state), host(lay.conv)
    worst = [0.0, 0.0]
    for t in range(wl.steps):
        S_ref, cs_ref, e = full_step_check(orc, lay, S_ref, cs_ref,
                                           kda_synth.step_inputs(wl, 0, t, DEV), 1e-5)
        worst = [max(a, b) for a, b in zip(worst, e)]
    say(f"tiny f32, 16 steps free-running: o {worst[0]:.3e} state {worst[1]:.3e}")


def test_tiny_bf16_teacher_forced(orc):
    wl = kda_synth.WORKLOADS["tiny"]
    lay = Layer(wl, 0, DEV, "bf16")
    S_free, cs_ref = host(lay.state), host(lay.conv)
    worst = [0.0, 0.0]
    for t in range(wl.steps):
        inp = kda_synth.step_inputs(wl, 0, t, DEV)
        cs_prev = cs_ref
        _, cs_ref, e = full_step_check(orc, lay, None, cs_ref, inp, 4e-3, teacher=True)
        worst = [max(a, b) for a, b in zip(worst, e)]
        S_free, _, _ = orc.decode_step(S_free, host(inp["x"]), host(lay.conv_w), cs_prev,
                                       host(inp["alpha"]), host(inp["beta"]), wl.scale)
    drift = rel_err(host(lay.state), S_free)
    say(f"tiny bf16, 16 steps teacher-forced: o {worst[0]:.3e} state {worst[1]:.3e}; "
        f"free-running drift vs double {drift:.3e} (reported, not gated)")


def test_tiny_matches_stored_fixture():
    """CPU-drawn tiny inputs, uploaded, against the stored oracle outputs."""
    from golden.make_tiny_fixture import OUT, tiny_inputs
    from hybrid_linear_attention_kda_amd import kda_decode_step
    wl, li, steps = tiny_inputs()
    stored = np.loadtxt(OUT, comments="#")
    o_ref = stored[:16 * 4 * 16].reshape(16, 1, 4, 16)
    S_ref = stored[16 * 4 * 16:].reshape(1, 4, 16, 16)
    dev = lambda a, dt: torch.from_numpy(a).to(DEV).to(dt)  # noqa: E731  exact: values are bf16/f32
    S = dev(li["state"], torch.float32)
    w = dev(li["conv_w"], torch.bfloat16)
    cs = dev(li["conv_state"], torch.bfloat16)
    o = torch.empty((1, 4, 16), dtype=torch.bfloat16, device=DEV)
    for t, s in enumerate(steps):
        kda_decode_step(S, dev(s["x"], torch.bfloat16), w, cs, cs, dev(s["alpha"], torch.float32),
                        dev(s["beta"], torch.float32), wl.scale, o)
        torch.cuda.synchronize()
        assert rel_err(host(o), o_ref[t]) <= TOL_O
    assert rel_err(host(S), S_ref) <= 1e-5


# ------------------------------------------------- GLM layer, one stream ----
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("inplace", [True, False], ids=["conv_inplace", "conv_pingpong"])
def test_glm_m1(orc, state_dtype, inplace):
    wl = kda_synth.WORKLOADS["glm_m1"]
    lay = Layer(wl, 0, DEV, state_dtype, inplace=inplace)
    S_ref, cs_ref = host(lay.state), host(lay.conv)
    _, _, e = full_step_check(orc, lay, S_ref, cs_ref, kda_synth.step_inputs(wl, 0, 0, DEV),
                              tol_state(state_dtype))
    say(f"glm_m1 {state_dtype} inplace={inplace}: o {e[0]:.3e} state {e[1]:.3e}")


# -------------------------------------------- M=8, 34 layers, one step -----
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_glm_m8_all_layers(orc, state_dtype):
    wl = kda_synth.WORKLOADS["glm_m8"]
    worst = [0.0, 0.0]
    for layer in range(wl.layers):
        lay = Layer(wl, layer, DEV, state_dtype)
        _, _, e = full_step_check(orc, lay, host(lay.state), host(lay.conv),
                                  kda_synth.step_inputs(wl, layer, 0, DEV), tol_state(state_dtype))
        worst = [max(a, b) for a, b in zip(worst, e)]
    say(f"glm_m8 {state_dtype}, 34 layers: o {worst[0]:.3e} state {worst[1]:.3e}")


# ------------------------------ M=32, 34 layers, 8 steps, f32 (headline) ----
def test_glm_m32_f32_full_and_sampled(orc):
    """Two layers compared in full over all 8 steps (free-running); every other
    layer on sampled (stream, head) units, also free-running over 8 steps."""
    wl = kda_synth.WORKLOADS["glm_m32"]
    rng = np.random.default_rng(32)
    worst = [0.0, 0.0]
    for layer in range(wl.layers):
        lay = Layer(wl, layer, DEV, "f32")
        if layer in (0, wl.layers - 1):
            S_ref, cs_ref = host(lay.state), host(lay.conv)
            for t in range(wl.steps):
                S_ref, cs_ref, e = full_step_check(orc, lay, S_ref, cs_ref,
                                                   kda_synth.step_inputs(wl, layer, t, DEV), 1e-5)
                worst = [max(a, b) for a, b in zip(worst, e)]
            continue
        units = [(int(rng.integers(wl.M)), int(rng.integers(wl.H))) for _ in range(3)]
        refs = {}
        for (m, h) in units:
            u = unit_inputs(wl, m, h, lay.conv_w, lay.conv)
            refs[(m, h)] = [host(lay.state[m, h]).reshape(1, 1, wl.D, wl.D), u["conv"], u["conv_w"]]
        for t in range(wl.steps):
            inp = kda_synth.step_inputs(wl, layer, t, DEV)
            lay.step(inp)
            torch.cuda.synchronize()
            for (m, h), r in refs.items():
                si = step_unit_inputs(wl, m, h, inp)
                r[0], r[1], o_ref = orc.decode_step(r[0], si["x"], r[2], r[1], si["alpha"],
                                                    si["beta"], wl.scale)
                e = (rel_err(host(lay.o[m, h]), o_ref[0, 0]), rel_err(host(lay.state[m, h]), r[0][0, 0]))
                assert e[0] <= TOL_O and e[1] <= 1e-5, f"layer {layer} step {t} unit {(m, h)}: {e}"
                worst = [max(a, b) for a, b in zip(worst, e)]
        del lay
    say(f"glm_m32 f32, 34 layers x 8 steps: o {worst[0]:.3e} state {worst[1]:.3e}")


# -------------------------- M=128, 34 layers, 8 steps, bf16 (serving) -------
def test_glm_m128_bf16_sampled_teacher_forced(orc):
    """Sampled units of every layer and step, including the pinned beta heads
    (0, 2^-24, 0.5, 1 - 2^-24, 1), teacher-forced from the GPU's bf16 state."""
    wl = kda_synth.WORKLOADS["glm_m128"]
    rng = np.random.default_rng(128)
    worst = [0.0, 0.0]
    for layer in range(wl.layers):
        lay = Layer(wl, layer, DEV, "bf16")
        m_tail = int(rng.integers(wl.M))
        units = [(m_tail, h) for h in range(len(kda_synth.BETA_TAILS))]
        units += [(int(rng.integers(wl.M)), int(rng.integers(wl.H))) for _ in range(2)]
        conv_ref = {}
        for (m, h) in units:
            u = unit_inputs(wl, m, h, lay.conv_w, lay.conv)
            conv_ref[(m, h)] = [u["conv"], u["conv_w"]]
        for t in range(wl.steps):
            inp = kda_synth.step_inputs(wl, layer, t, DEV)
            S_prev = {mh: host(lay.state[mh[0], mh[1]]).reshape(1, 1, wl.D, wl.D) for mh in units}
            lay.step(inp)
            torch.cuda.synchronize()
            for (m, h) in units:
                si = step_unit_inputs(wl, m, h, inp)
                cs, w = conv_ref[(m, h)]
                S_ref, conv_ref[(m, h)][0], o_ref = orc.decode_step(
                    S_prev[(m, h)], si["x"], w, cs, si["alpha"], si["beta"], wl.scale)
                e = (rel_err(host(lay.o[m, h]), o_ref[0, 0]), rel_err(host(lay.state[m, h]), S_ref[0, 0]))
                assert e[0] <= TOL_O and e[1] <= 4e-3, f"layer {layer} step {t} unit {(m, h)}: {e}"
                worst = [max(a, b) for a, b in zip(worst, e)]
        del lay
    say(f"glm_m128 bf16, 34 layers x 8 steps sampled: o {worst[0]:.3e} state {worst[1]:.3e}")


# ------------------------------------------------------- ragged shapes ------
@pytest.mark.parametrize("M,H,D", [(3, 5, 128), (5, 3, 64), (7, 2, 32), (2, 7, 16), (1, 1, 128),
                                   (9, 1, 16)])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_ragged_shapes(orc, M, H, D, state_dtype):
    wl = kda_synth.custom(f"ragged_{M}_{H}_{D}", M, H, D, steps=3)
    for inplace in (True, False):
        lay = Layer(wl, 0, DEV, state_dtype, inplace=inplace)
        S_ref, cs_ref = host(lay.state), host(lay.conv)
        for t in range(wl.steps):
            inp = kda_synth.step_inputs(wl, 0, t, DEV)
            S_ref, cs_ref, _ = full_step_check(orc, lay, S_ref, cs_ref, inp, tol_state(state_dtype),
                                               teacher=state_dtype == "bf16")


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("inplace", [True, False], ids=["conv_inplace", "conv_pingpong"])
def test_many_units_ragged(orc, state_dtype, inplace):
    """M*H = 1600 heads: the whole-head launch at a size that is not a multiple
    of 8, so the last workgroups of the grid cover a ragged tail of heads."""
    wl = kda_synth.custom("many_units", 25, 64, 128, steps=3)
    lay = Layer(wl, 0, DEV, state_dtype, inplace=inplace)
    S_ref, cs_ref = host(lay.state), host(lay.conv)
    for t in range(wl.steps):
        S_ref, cs_ref, e = full_step_check(orc, lay, S_ref, cs_ref,
                                           kda_synth.step_inputs(wl, 0, t, DEV), tol_state(state_dtype),
                                           teacher=state_dtype == "bf16")
    say(f"many units {state_dtype} inplace={inplace}: o {e[0]:.3e} state {e[1]:.3e}")


@pytest.mark.parametrize("M,H", [(33, 64), (33, 63)])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_wide_grid_whole_tensors(orc, state_dtype, M, H):
    """33 x 64 = 2112 and 33 x 63 = 2079 heads, whole tensors: from 2048 heads
    on, the whole-head launches store the state through agent-scope buffer
    stores instead of global stores, and neither count is a multiple of the
    CU count, so the last round of workgroups is partial.  The 16-wave f32
    grid takes consecutive workgroups alternately from the two halves of the
    heads when their number is even (2112) and in order when it is odd
    (2079); every head must be updated exactly once either way."""
    wl = kda_synth.custom("wide", M, H, 128, steps=2)
    lay = Layer(wl, 0, DEV, state_dtype)
    S_ref, cs_ref = host(lay.state), host(lay.conv)
    for t in range(wl.steps):
        S_ref, cs_ref, e = full_step_check(orc, lay, S_ref, cs_ref,
                                           kda_synth.step_inputs(wl, 0, t, DEV), tol_state(state_dtype),
                                           teacher=state_dtype == "bf16")
    say(f"wide grid {M}x{H} {state_dtype}: o {e[0]:.3e} state {e[1]:.3e}")


def test_empty_batch():
    from hybrid_linear_attention_kda_amd import kda_decode_step
    e = lambda *s, dt=torch.float32: torch.empty(s, dtype=dt, device=DEV)  # noqa: E731
    H, D = 4, 16
    kda_decode_step(e(0, H, D, D), e(0, 3, H * D, dt=torch.bfloat16), e(3 * H * D, 4, dt=torch.bfloat16),
                    e(0, 3, 3 * H * D, dt=torch.bfloat16), e(0, 3, 3 * H * D, dt=torch.bfloat16),
                    e(0, H, D), e(0, H), 1.0, e(0, H, D, dt=torch.bfloat16))
    torch.cuda.synchronize()
