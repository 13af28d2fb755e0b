"""GPU parity of kda_decode_multi (T tokens per stream in one call) against
the CPU oracle's T consecutive steps ("GLM-5.3 deep dive" 8.2.6).

The state stays on chip for all T tokens, so f32 state is compared
free-running (1e-5) and bf16 state sees one rounding per call (4e-3);
every token's output is checked (4e-3)."""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from hybrid_linear_attention_kda_amd import kda_decode_multi, kda_decode_step
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


def tokens(wl, layer, T, t0=0):
    """Per-token inputs stacked along a token axis: x [M,T,3,HD], alpha [M,T,H,D], beta [M,T,H]."""
    steps = [kda_synth.step_inputs(wl, layer, t0 + t, DEV) for t in range(T)]
    return {k: torch.stack([s[k] for s in steps], dim=1).contiguous() for k in ("x", "alpha", "beta")}


def run_multi(wl, state_dtype, T, inplace, layer=0):
    li = kda_synth.layer_inputs(wl, layer, DEV, state_dtype)
    S, w, cs = li["state"], li["conv_w"], li["conv_state"]
    cout = cs if inplace else torch.empty_like(cs)
    ins = tokens(wl, layer, T)
    o = torch.empty((wl.M, T, wl.H, wl.D), dtype=torch.bfloat16, device=DEV)
    S0, cs0 = host(S), host(cs)
    kda_decode_multi(S, ins["x"], w, cs, cout, ins["alpha"], ins["beta"], wl.scale, o)
    torch.cuda.synchronize()
    return S0, cs0, li, ins, S, cout, o


@pytest.mark.parametrize("inplace", [True, False], ids=["conv_inplace", "conv_pingpong"])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,H,D,T", [(1, 4, 16, 16), (2, 3, 32, 5), (3, 2, 64, 3), (3, 5, 128, 7),
                                     (8, 64, 128, 8), (2, 64, 128, 1), (1, 1, 128, 64)])
def test_multi_against_oracle(orc, M, H, D, T, state_dtype, inplace):
    wl = kda_synth.WORKLOADS["tiny"] if (M, H, D) == (1, 4, 16) else kda_synth.custom(
        f"multi_{M}_{H}_{D}", M, H, D, steps=T)
    S0, cs0, li, ins, S, cout, o = run_multi(wl, state_dtype, T, inplace)
    S_ref, cs_ref, o_ref = orc.decode_multi(S0, host(ins["x"]), host(li["conv_w"]), cs0,
                                            host(ins["alpha"]), host(ins["beta"]), wl.scale)
    assert np.array_equal(host(cout), cs_ref), "conv state after T tokens"
    e_s = rel_err(host(S), S_ref)
    e_o = max(rel_err(host(o[:, t]), o_ref[:, t]) for t in range(T))
    say(f"multi ({M},{H},{D}) T={T} {state_dtype}: state {e_s:.3e} o {e_o:.3e}")
    assert e_s <= tol_state(state_dtype), f"state error {e_s:.3e}"
    assert e_o <= TOL_O, f"output error {e_o:.3e}"


@pytest.mark.parametrize("M,H,D,T", [(4, 64, 128, 8), (3, 5, 64, 6)])
def test_multi_equals_single_steps_f32(M, H, D, T):
    """One multi-token call and T single-token calls agree to f32 rounding."""
    wl = kda_synth.custom(f"multi_vs_single_{M}_{D}", M, H, D, steps=T)
    _, _, li, ins, S, cout, o = run_multi(wl, "f32", T, True)
    li2 = kda_synth.layer_inputs(wl, 0, DEV, "f32")
    S2, cs2 = li2["state"], li2["conv_state"]
    o2 = torch.empty((M, H, D), dtype=torch.bfloat16, device=DEV)
    for t in range(T):
        kda_decode_step(S2, ins["x"][:, t].contiguous(), li2["conv_w"], cs2, cs2,
                        ins["alpha"][:, t].contiguous(), ins["beta"][:, t].contiguous(), wl.scale, o2)
        torch.cuda.synchronize()
        assert rel_err(host(o[:, t]), host(o2)) <= 2 ** -7, f"token {t}"
    assert torch.equal(cout, cs2)
    assert rel_err(host(S), host(S2)) <= 2e-6


@pytest.mark.parametrize("state_dtype,T", [("f32", 8), ("f32", 5), ("bf16", 8), ("f32", 12), ("bf16", 20)])
def test_multi_wide_grid_whole_tensors(orc, state_dtype, T):
    """33 x 64 = 2112 heads, whole tensors: from 2048 heads on the chunk form
    stores the state with agent scope (buffer stores over each head's
    bytes), both in the one-chunk launch (T = 8; f32 T = 5 and 8 in the
    staggered form, whose odd workgroups request their state after the
    coefficients) and after the chunk loop (T = 12, 20); 2112 is not a
    multiple of the CU count."""
    wl = kda_synth.custom("multi_wide", 33, 64, 128, steps=T)
    S0, cs0, li, ins, S, cout, o = run_multi(wl, state_dtype, T, False)
    S_ref, cs_ref, o_ref = orc.decode_multi(S0, host(ins["x"]), host(li["conv_w"]), cs0,
                                            host(ins["alpha"]), host(ins["beta"]), wl.scale)
    assert np.array_equal(host(cout), cs_ref), "conv state after T tokens"
    e_s = rel_err(host(S), S_ref)
    e_o = max(rel_err(host(o[:, t]), o_ref[:, t]) for t in range(T))
    say(f"multi wide T={T} {state_dtype}: state {e_s:.3e} o {e_o:.3e}")
    assert e_s <= tol_state(state_dtype), f"state error {e_s:.3e}"
    assert e_o <= TOL_O, f"output error {e_o:.3e}"


def test_multi_glm_m32_sampled(orc):
    """The benchmark's multi-token launch (M = 32, T = 8, FP32 state) on
    sampled (stream, head) units against the oracle."""
    wl = kda_synth.WORKLOADS["glm_m32"]
    T = 8
    S0, cs0, li, ins, S, cout, o = run_multi(wl, "f32", T, True)
    H, D = wl.H, wl.D
    cw = host(li["conv_w"]).reshape(3, H, D, 4)
    for (m, h) in [(0, 0), (5, 17), (31, 63), (20, 33)]:
        S_ref, _, o_ref = orc.decode_multi(
            S0[m, h][None, None], host(ins["x"][m]).reshape(T, 3, H, D)[:, :, h].reshape(1, T, 3, D),
            cw[:, h].reshape(3 * D, 4), cs0[m].reshape(3, 3, H, D)[:, :, h].reshape(1, 3, 3 * D),
            host(ins["alpha"][m, :, h])[None, :, None], host(ins["beta"][m, :, h])[None, :, None], wl.scale)
        assert rel_err(host(S[m, h]), S_ref[0, 0]) <= 1e-5, f"state ({m},{h})"
        assert rel_err(host(o[m, :, h]), o_ref[0, :, 0]) <= TOL_O, f"outputs ({m},{h})"
    say("multi glm_m32 T=8 sampled units ok")


def test_multi_empty():
    wl = kda_synth.custom("multi_empty", 2, 3, 16)
    li = kda_synth.layer_inputs(wl, 0, DEV, "f32")
    S = li["state"].clone()
    e = lambda *s, dt=torch.float32: torch.empty(s, dtype=dt, device=DEV)  # noqa: E731
    kda_decode_multi(S, e(2, 0, 3, 48, dt=torch.bfloat16), li["conv_w"], li["conv_state"], li["conv_state"],
                     e(2, 0, 3, 16), e(2, 0, 3), 0.25, e(2, 0, 3, 16, dt=torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(S, li["state"])


# Fade extremes: alpha of exactly 1, a steep fade whose running product
# underflows f32 within a few tokens, tokens with alpha 1e-25 or exactly 0 in
# some rows, and alpha log-uniform over [1e-9, 1] -- over enough tokens to
# cross many of the kernel's token chunks.  Any scheme that reorders or defers
# the per-row fade must still match the oracle's plain recurrence on these.
def fade_pattern(case, M, T, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    if case == "one":
        a = torch.ones(M, T, H, D, dtype=torch.float64)
    elif case == "steep":                  # C passes 2^-64 every few tokens
        a = torch.full((M, T, H, D), 2.0 ** -12, dtype=torch.float64)
    elif case == "tiny":                   # chunks whose own product underflows the range
        a = torch.rand(M, T, H, D, generator=g, dtype=torch.float64) * 0.5 + 0.5
        a[:, 3::7] = 1e-25
    elif case == "zero":                   # some rows reset outright
        a = torch.rand(M, T, H, D, generator=g, dtype=torch.float64) * 0.5 + 0.5
        a[:, 5::9, :, ::3] = 0.0
    else:                                  # log-uniform over [1e-9, 1]
        a = torch.exp(-torch.rand(M, T, H, D, generator=g, dtype=torch.float64) * (9 * np.log(10)))
    return a.float().to(DEV).contiguous()


@pytest.mark.parametrize("case", ["one", "steep", "tiny", "zero", "loguniform"])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,H,D,T", [(2, 3, 128, 40), (2, 2, 64, 33), (1, 2, 16, 29)])
def test_multi_fade_extremes(orc, M, H, D, T, state_dtype, case):
    wl = kda_synth.custom(f"multi_fade_{M}_{H}_{D}", M, H, D, steps=T)
    li = kda_synth.layer_inputs(wl, 0, DEV, state_dtype)
    S, w, cs = li["state"], li["conv_w"], li["conv_state"]
    ins = tokens(wl, 0, T)
    alpha = fade_pattern(case, M, T, H, D, seed=D + T)
    o = torch.empty((M, T, H, D), dtype=torch.bfloat16, device=DEV)
    S0, cs0 = host(S), host(cs)
    kda_decode_multi(S, ins["x"], w, cs, cs, alpha, ins["beta"], wl.scale, o)
    torch.cuda.synchronize()
    S_ref, cs_ref, o_ref = orc.decode_multi(S0, host(ins["x"]), host(w), cs0, host(alpha), host(ins["beta"]),
                                            wl.scale)
    assert torch.isfinite(S).all() and torch.isfinite(o.float()).all()
    assert np.array_equal(host(cs), cs_ref)
    e_s = rel_err(host(S), S_ref)
    e_o = max(rel_err(host(o[:, t]), o_ref[:, t]) for t in range(T))
    say(f"multi fade {case} ({M},{H},{D}) T={T} {state_dtype}: state {e_s:.3e} o {e_o:.3e}")
    assert e_s <= tol_state(state_dtype), f"state error {e_s:.3e}"
    assert e_o <= TOL_O, f"output error {e_o:.3e}"


# Token counts around the D = 128 kernel's 8-token chunks: one chunk plus one
# token, two full chunks, two plus one, and a ragged third; and on both sides
# of the T at which the bf16 state switches between the token loop and the
# chunk form (4 | 5, 11 | 12, 18 | 19).
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [4, 5, 9, 11, 12, 16, 17, 18, 19, 23])
def test_multi_chunk_boundaries(orc, T, state_dtype):
    M, H, D = 2, 3, 128
    wl = kda_synth.custom(f"multi_bound_{T}", M, H, D, steps=T)
    S0, cs0, li, ins, S, cout, o = run_multi(wl, state_dtype, T, inplace=False)
    S_ref, cs_ref, o_ref = orc.decode_multi(S0, host(ins["x"]), host(li["conv_w"]), cs0,
                                            host(ins["alpha"]), host(ins["beta"]), wl.scale)
    assert np.array_equal(host(cout), cs_ref), "conv state after T tokens"
    e_s = rel_err(host(S), S_ref)
    e_o = max(rel_err(host(o[:, t]), o_ref[:, t]) for t in range(T))
    say(f"multi chunk boundary T={T} {state_dtype}: state {e_s:.3e} o {e_o:.3e}")
    assert e_s <= tol_state(state_dtype), f"state error {e_s:.3e}"
    assert e_o <= TOL_O, f"output error {e_o:.3e}"
