"""GPU parity of kda_prefill_gated_ws, the two-pass chunk form of "GLM-5.3
deep dive" 8.2.5 (pass 1: every chunk's intra-chunk work in parallel,
written to a caller workspace; pass 2: the state carried through the chunks
in order), against the CPU oracle's token-by-token gated recurrence.

Tolerances as the one-pass prefill's (relative to the largest reference
magnitude): f32 state 1e-5, bf16 state 4e-3 (one rounding, at the end of the
call however many segments run), outputs 4e-3.  The two passes perform the
one-pass kernel's operations per chunk, except that W S is summed over the
four 32-row blocks of the state as four partial sums (independent MFMA
chains) rather than one running sum, so the two forms agree to f32 rounding,
not bit for bit; a segmented two-pass call carries the state between
segments in f32 and is bit-identical to a one-segment call.
"""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from hybrid_linear_attention_kda_amd import kda_prefill_gated, kda_prefill_workspace_bytes
from kda_gpu_util import TOL_O, host, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_STATE_PREFILL = 1e-5
REC = 42496            # KDA_PREFILL_RECORD_BYTES
STAGE = 128 * 128 * 4  # f32 copy of one head's state (bf16 storage, segmented calls)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def say(msg):
    print(msg, flush=True)


def sequence(wl, L, layer=0):
    st = [kda_synth.step_inputs(wl, layer, t, DEV) for t in range(L)]
    gi = [kda_synth.gate_inputs(wl, layer, t, DEV) for t in range(L)]
    return (torch.stack([s["x"] for s in st], 1).contiguous(),
            torch.stack([g["f"] for g in gi], 1).contiguous(),
            torch.stack([g["beta_logit"] for g in gi], 1).contiguous())


def workspace(M, H, L, state_dtype, mode):
    """full: one segment; chunks_k: records of k chunks (the sequence then
    runs in segments of k chunks), plus the f32 state stage for bf16."""
    if mode == "full":
        n = kda_prefill_workspace_bytes(L, M, H, 128)
    else:
        k = int(mode.split("_")[1])
        n = k * M * H * REC
        if state_dtype == "bf16" and k < (L + 15) // 16:
            n += M * H * STAGE
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def run_ws(M, H, L, state_dtype, lb, inplace, name, mode, passes=2, seed=100):
    wl = kda_synth.custom(name, M, H, 128, steps=max(L, 1), seed=seed)
    li = kda_synth.layer_inputs(wl, 0, DEV, state_dtype)
    gp = kda_synth.gate_params(wl, 0, DEV)
    S, w, cs = li["state"], li["conv_w"], li["conv_state"]
    cout = cs if inplace else torch.empty_like(cs)
    x, f, bl = sequence(wl, L)
    o = torch.empty((M, L, H, 128), dtype=torch.bfloat16, device=DEV)
    S0, cs0 = host(S), host(cs)
    ws = workspace(M, H, L, state_dtype, mode) if passes != 1 else None
    kda_prefill_gated(S, x, w, cs, cout, f, gp["A_log"], gp["dt_bias"], bl, wl.scale, o, lower_bound=lb,
                      workspace=ws, passes=passes)
    torch.cuda.synchronize()
    return wl, gp, (x, f, bl), S, cout, o, S0, cs0, w


SHAPES = [(1, 1, 16), (1, 2, 37), (2, 3, 64), (1, 4, 100), (1, 1, 1), (2, 2, 3)]


@pytest.mark.parametrize("mode", ["full", "chunks_1", "chunks_3"])
@pytest.mark.parametrize("inplace", [True, False], ids=["conv_inplace", "conv_pingpong"])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,H,L", SHAPES)
def test_two_pass_against_oracle(orc, M, H, L, state_dtype, inplace, mode):
    lb = -5.0 if (M + H + L) % 2 else -1.5
    wl, gp, (x, f, bl), S, cout, o, S0, cs0, w = run_ws(M, H, L, state_dtype, lb, inplace,
                                                        f"prefill_ws_{M}_{H}_{L}", mode)
    S_ref, cs_ref, o_ref = orc.sequence_gated(S0, host(x), host(w), cs0, host(f), host(gp["A_log"]),
                                              host(gp["dt_bias"]), host(bl), wl.scale, lower_bound=lb)
    assert np.array_equal(host(cout), cs_ref), "conv state after the sequence"
    e_s = rel_err(host(S), S_ref)
    e_o = max(rel_err(host(o[:, t]), o_ref[:, t]) for t in range(L))
    say(f"two-pass ({M},{H},L={L}) {state_dtype} {mode} inplace={inplace}: state {e_s:.3e} o {e_o:.3e}")
    assert e_s <= (TOL_STATE_PREFILL if state_dtype == "f32" else 4e-3), f"state error {e_s:.3e}"
    assert e_o <= TOL_O, f"output error {e_o:.3e}"


@pytest.mark.parametrize("M,H,L,state_dtype,mode", [
    (1, 64, 300, "f32", "full"), (1, 64, 300, "f32", "chunks_2"), (2, 3, 64, "bf16", "full"),
    (2, 3, 100, "bf16", "chunks_1"), (1, 1, 1, "f32", "full"), (3, 2, 17, "f32", "chunks_1"),
    (1, 5, 35, "bf16", "chunks_2"), (4, 64, 48, "f32", "full")])
def test_two_pass_matches_one_pass(M, H, L, state_dtype, mode):
    """Same inputs through the one-pass kernel, the two passes with a whole
    workspace and the two passes with `mode`'s workspace: the two-pass
    results agree with the one-pass ones to f32 rounding (state 1e-6 for
    f32 storage, one bf16 ulp of the largest value for bf16 storage and
    outputs) and are bit-identical between the workspace sizes; conv states
    are bit-identical."""
    tag = f"prefill_eq_{M}_{H}_{L}"
    r1 = run_ws(M, H, L, state_dtype, -5.0, False, tag, mode, passes=1, seed=5)
    rf = run_ws(M, H, L, state_dtype, -5.0, False, tag, "full", passes=2, seed=5)
    r2 = run_ws(M, H, L, state_dtype, -5.0, False, tag, mode, passes=2, seed=5)
    assert torch.equal(rf[3], r2[3]) and torch.equal(rf[5], r2[5]), "segmented = one segment, bit for bit"
    assert torch.equal(r1[4], r2[4]), "conv state"
    e_s = rel_err(host(r2[3]), host(r1[3]))
    e_o = rel_err(host(r2[5]), host(r1[5]))
    assert e_s <= (1e-6 if state_dtype == "f32" else 2 ** -8), f"state {e_s:.3e}"
    assert e_o <= 2 ** -8, f"outputs {e_o:.3e}"
    say(f"two-pass ({M},{H},L={L}) {state_dtype} {mode}: state {e_s:.3e} o {e_o:.3e} against one pass")


def test_two_pass_empty():
    wl = kda_synth.custom("prefill_ws_empty", 1, 2, 128)
    li = kda_synth.layer_inputs(wl, 0, DEV, "f32")
    gp = kda_synth.gate_params(wl, 0, DEV)
    S = li["state"].clone()
    e = lambda *s, dt=torch.bfloat16: torch.empty(s, dtype=dt, device=DEV)  # noqa: E731
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    kda_prefill_gated(S, e(1, 0, 3, 256), li["conv_w"], li["conv_state"], li["conv_state"], e(1, 0, 256),
                      gp["A_log"], gp["dt_bias"], e(1, 0, 2), wl.scale, e(1, 0, 2, 128), workspace=ws, passes=2)
    torch.cuda.synchronize()
    assert torch.equal(S, li["state"])


@pytest.mark.parametrize("case", ["saturated_gate", "beta_extremes"])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_two_pass_gate_extremes(orc, case, state_dtype):
    """The one-pass tests' extremes (a chunk decaying by e^-80; beta ~ 0 and
    ~ 1) through two passes in 2-chunk segments."""
    M, H, L, D = 2, 3, 53, 128
    wl = kda_synth.custom(f"prefill_ext_{case}", M, H, D, steps=L, seed=11)
    li = kda_synth.layer_inputs(wl, 0, DEV, state_dtype)
    gp = kda_synth.gate_params(wl, 0, DEV)
    x, f, bl = sequence(wl, L)
    if case == "saturated_gate":
        gp["dt_bias"] = torch.full_like(gp["dt_bias"], 12.0)
    else:
        sign = torch.where(torch.arange(L, device=DEV) % 2 == 0, 1.0, -1.0)
        bl = (20.0 * sign)[None, :, None].expand(M, L, H).to(torch.bfloat16).contiguous()
    S, cs = li["state"], li["conv_state"]
    o = torch.empty((M, L, H, D), dtype=torch.bfloat16, device=DEV)
    S0, cs0 = host(S), host(cs)
    ws = workspace(M, H, L, state_dtype, "chunks_2")
    kda_prefill_gated(S, x, li["conv_w"], cs, cs, f, gp["A_log"], gp["dt_bias"], bl, wl.scale, o,
                      workspace=ws, passes=2)
    torch.cuda.synchronize()
    S_ref, cs_ref, o_ref = orc.sequence_gated(S0, host(x), host(li["conv_w"]), cs0, host(f), host(gp["A_log"]),
                                              host(gp["dt_bias"]), host(bl), wl.scale)
    assert torch.isfinite(S).all() and torch.isfinite(o.float()).all()
    e_s = rel_err(host(S), S_ref)
    e_o = max(rel_err(host(o[:, t]), o_ref[:, t]) for t in range(L))
    say(f"two-pass {case} {state_dtype}: state {e_s:.3e} o {e_o:.3e}")
    assert np.array_equal(host(cs), cs_ref)
    assert e_s <= (TOL_STATE_PREFILL if state_dtype == "f32" else 4e-3), f"state error {e_s:.3e}"
    assert e_o <= TOL_O, f"output error {e_o:.3e}"


# The benchmark's two-pass prefill shapes, inputs and launch (bench.py's
# measure_prefill: workload prefill_m{M}_l{L}, seed 7, whole-sequence draws,
# lower bound -5, conv state ping-pong, the library's choice of form with a
# one-segment workspace), on sampled (stream, head) units over every token.
WS_BENCH_SHAPES = [(1, 8192, "f32"), (2, 4096, "f32"), (1, 4096, "bf16")]


@pytest.mark.parametrize("M,L,state_dtype", WS_BENCH_SHAPES)
def test_two_pass_benchmark_shapes_sampled(orc, M, L, state_dtype):
    H, D = 64, 128
    wl = kda_synth.custom(f"prefill_m{M}_l{L}", M, H, D, steps=L, seed=7)
    li = kda_synth.layer_inputs(wl, 0, DEV, state_dtype)
    gp = kda_synth.gate_params(wl, 0, DEV)
    seq = kda_synth.sequence_inputs(wl, 0, L, DEV)
    S, cs = li["state"], li["conv_state"]
    cout = torch.empty_like(cs)
    o = torch.empty((M, L, H, D), dtype=torch.bfloat16, device=DEV)
    units = sorted({(0, 0), (M - 1, H - 1), (M // 2, 17), (min(1, M - 1), 40)})
    S0 = {u: host(S[u[0], u[1]]) for u in units}
    cs0 = host(cs)
    ws = workspace(M, H, L, state_dtype, "full")
    kda_prefill_gated(S, seq["x"], li["conv_w"], cs, cout, seq["f"], gp["A_log"], gp["dt_bias"],
                      seq["beta_logit"], wl.scale, o, workspace=ws, passes=0)
    torch.cuda.synchronize()
    cw = host(li["conv_w"]).reshape(3, H, D, 4)
    tol_s = TOL_STATE_PREFILL if state_dtype == "f32" else 4e-3
    worst_s = worst_o = 0.0
    for (m, h) in units:
        sl = slice(h * D, (h + 1) * D)
        xu = host(seq["x"][m, :, :, sl]).reshape(1, L, 3, D)
        S_ref, cs_ref, o_ref = orc.sequence_gated(
            S0[(m, h)][None, None], xu, cw[:, h].reshape(3 * D, 4),
            cs0[m].reshape(3, 3, H, D)[:, :, h].reshape(1, 3, 3 * D),
            host(seq["f"][m, :, sl])[None], host(gp["A_log"][h:h + 1]), host(gp["dt_bias"][sl]),
            host(seq["beta_logit"][m, :, h:h + 1])[None], wl.scale)
        assert np.array_equal(host(cout[m]).reshape(3, 3, H, D)[:, :, h].reshape(3, 3 * D), cs_ref[0]), \
            f"conv state ({m},{h})"
        e_s = rel_err(host(S[m, h]), S_ref[0, 0])
        e_o = rel_err(host(o[m, :, h]), o_ref[0, :, 0])
        worst_s, worst_o = max(worst_s, e_s), max(worst_o, e_o)
        assert e_s <= tol_s, f"state ({m},{h}): {e_s:.3e}"
        assert e_o <= TOL_O, f"outputs ({m},{h}): {e_o:.3e}"
    say(f"two-pass {M} x {L} tokens {state_dtype}, units {units}: state {worst_s:.3e} o {worst_o:.3e}")
