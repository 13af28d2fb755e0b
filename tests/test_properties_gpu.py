"""GPU properties of the HIP path that hold at any size: determinism, split and
stream independence, fused == conv + recurrent, checkpoint/resume, and the
special cases the method has (identity, zero input, exact recall)."""
import numpy as np
import pytest
import torch

import kda_synth
import oracle
from hybrid_linear_attention_kda_amd import kda_conv_step, kda_decode_step, kda_recurrent_step
from kda_gpu_util import TOL_O, Layer, host, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def run(wl, state_dtype, steps, nsplit=None, inplace=True, stream=None):
    lay = Layer(wl, 0, DEV, state_dtype, inplace=inplace)
    outs = []
    for t in range(steps):
        lay.step(kda_synth.step_inputs(wl, 0, t, DEV), nsplit=nsplit, stream=stream)
        outs.append(lay.o.clone())
    torch.cuda.synchronize()
    return lay, outs


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [4, 32])
def test_bitwise_deterministic(state_dtype, M):
    wl = kda_synth.custom("det", M, 64, 128, steps=3)
    a, oa = run(wl, state_dtype, 3)
    b, ob = run(wl, state_dtype, 3)
    assert torch.equal(a.state, b.state) and all(torch.equal(x, y) for x, y in zip(oa, ob))


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_split_agrees_to_rounding(orc, state_dtype):
    """Splitting a head's value columns over 2 or 4 workgroups changes only the
    order of the f32 sums over key rows: the conv state is bit-identical, the
    state and output agree to f32 rounding (plus one bf16 ulp where stored as
    bf16), and every split matches the oracle."""
    wl = kda_synth.custom("split", 2, 64, 128, steps=1)
    ref, oref = run(wl, state_dtype, 1, nsplit=1, inplace=False)
    S0 = host(kda_synth.initial_state(wl, 0, DEV, state_dtype))
    lay0 = Layer(wl, 0, DEV, state_dtype)
    inp = kda_synth.step_inputs(wl, 0, 0, DEV)
    S_ref, _, o_ref = orc.decode_step(S0, host(inp["x"]), host(lay0.conv_w), host(lay0.conv),
                                      host(inp["alpha"]), host(inp["beta"]), wl.scale)
    tol_s = 1e-6 if state_dtype == "f32" else 2 ** -7
    for ns in (2, 4):
        lay, outs = run(wl, state_dtype, 1, nsplit=ns, inplace=False)
        assert torch.equal(lay.conv, ref.conv), f"nsplit={ns} conv state"
        assert rel_err(host(lay.state), host(ref.state)) <= tol_s, f"nsplit={ns} state"
        assert rel_err(host(outs[0]), host(oref[0])) <= 2 ** -7, f"nsplit={ns} output"
        assert rel_err(host(outs[0]), o_ref) <= TOL_O
        assert rel_err(host(lay.state), S_ref) <= (1e-5 if state_dtype == "f32" else 4e-3)


@pytest.mark.parametrize("entry", ["plain", "gated", "layer"])
def test_store_policy_bitwise_bf16(entry):
    """bf16 state: the same whole-head kernel runs below and above 2048 heads;
    only the state store's cache policy differs (agent scope from 2048 heads
    on).  32 streams (2048 heads) and their first 31 (1984 heads) in a call of
    their own must agree bit for bit on those 31 streams."""
    from hybrid_linear_attention_kda_amd import (KDA_GATE_BOUNDED, kda_decode_layer_step,
                                                 kda_decode_step_gated)
    M, H, D = 32, 64, 128
    wl = kda_synth.custom("policy", M, H, D, steps=1)
    li = kda_synth.layer_inputs(wl, 0, DEV, "bf16")
    inp = kda_synth.step_inputs(wl, 0, 0, DEV)
    gp = kda_synth.gate_params(wl, 0, DEV)
    gi = kda_synth.gate_inputs(wl, 0, 0, DEV)
    outs = []
    for m in (M, M - 1):
        S = li["state"][:m].clone()
        cs = li["conv_state"][:m].clone()
        o = torch.empty((m, H, D), dtype=torch.bfloat16, device=DEV)
        if entry == "plain":
            kda_decode_step(S, inp["x"][:m], li["conv_w"], cs, cs, inp["alpha"][:m], inp["beta"][:m],
                            wl.scale, o)
        elif entry == "gated":
            kda_decode_step_gated(S, inp["x"][:m], li["conv_w"], cs, cs, gi["f"][:m], gp["A_log"],
                                  gp["dt_bias"], gi["beta_logit"][:m], wl.scale, o,
                                  gate_kind=KDA_GATE_BOUNDED, lower_bound=-5.0)
        else:
            kda_decode_layer_step(S, inp["x"][:m], li["conv_w"], cs, cs, gi["f"][:m], gp["A_log"],
                                  gp["dt_bias"], gi["beta_logit"][:m], wl.scale, gi["out_gate"][:m],
                                  gp["norm_w"], o, gate_kind=KDA_GATE_BOUNDED, lower_bound=-5.0)
        outs.append((S, cs, o))
    torch.cuda.synchronize()
    (S1, c1, o1), (S2, c2, o2) = outs
    n = M - 1
    assert torch.equal(S1[:n], S2) and torch.equal(c1[:n], c2) and torch.equal(o1[:n], o2)


def test_packed_bf16_equals_unpacked():
    """bf16 state, plain step: up to 8 heads per CU (2048 on 256 CUs) the
    kernel keeps the state in its packed registers and unpacks each row
    twice; above, it holds the rows as f32.  Both form the same products in
    the same order: 33 streams (2112 heads, the unpacked form) and their
    first 32 (2048 heads, the packed form) agree bit for bit on those 32."""
    M, H, D = 33, 64, 128
    wl = kda_synth.custom("packed", M, H, D, steps=2)
    li = kda_synth.layer_inputs(wl, 0, DEV, "bf16")
    res = []
    for m in (M, M - 1):
        S = li["state"][:m].clone()
        cs = li["conv_state"][:m].clone()
        o = torch.empty((m, H, D), dtype=torch.bfloat16, device=DEV)
        outs = []
        for t in range(2):
            inp = kda_synth.step_inputs(wl, 0, t, DEV)
            kda_decode_step(S, inp["x"][:m], li["conv_w"], cs, cs, inp["alpha"][:m], inp["beta"][:m],
                            wl.scale, o)
            outs.append(o.clone())
        res.append((S, cs, outs))
    torch.cuda.synchronize()
    (S1, c1, o1), (S2, c2, o2) = res
    n = M - 1
    assert torch.equal(S1[:n], S2) and torch.equal(c1[:n], c2)
    assert all(torch.equal(a[:n], b) for a, b in zip(o1, o2))


def test_inplace_conv_equals_pingpong():
    wl = kda_synth.custom("pp", 3, 8, 128, steps=4)
    a, oa = run(wl, "f32", 4, nsplit=1, inplace=True)
    b, ob = run(wl, "f32", 4, nsplit=1, inplace=False)
    assert torch.equal(a.state, b.state) and torch.equal(a.conv, b.conv)
    assert all(torch.equal(x, y) for x, y in zip(oa, ob))


def test_side_stream_equals_default_stream():
    wl = kda_synth.custom("stream", 2, 16, 128, steps=2)
    a, oa = run(wl, "f32", 2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b, ob = run(wl, "f32", 2, stream=s)
    s.synchronize()
    assert torch.equal(a.state, b.state) and all(torch.equal(x, y) for x, y in zip(oa, ob))


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,H,D", [(3, 8, 16), (3, 8, 128), (16, 64, 128), (32, 64, 128)])
def test_fused_equals_conv_then_recurrent(state_dtype, M, H, D):
    """Bitwise, when both paths get the same work split: the fused call uses
    distinct conv buffers so that, like the recurrent entry, it may split a
    head when M*H is small."""
    wl = kda_synth.custom("unfused", M, H, D, steps=2)
    fused = Layer(wl, 0, DEV, state_dtype, inplace=False)
    split = Layer(wl, 0, DEV, state_dtype)
    C = 3 * wl.H * D
    y = torch.empty((wl.M, C), dtype=torch.float32, device=DEV)
    for t in range(wl.steps):
        inp = kda_synth.step_inputs(wl, 0, t, DEV)
        fused.step(inp)
        kda_conv_step(inp["x"].view(wl.M, C), split.conv_w, split.conv.view(wl.M, 3, C),
                      split.conv.view(wl.M, 3, C), y)
        kda_recurrent_step(split.state, y.view(wl.M, 3, wl.H * D), inp["alpha"], inp["beta"],
                           wl.scale, split.o)
        torch.cuda.synchronize()
        assert torch.equal(fused.o, split.o)
        assert torch.equal(fused.state, split.state)
        assert torch.equal(fused.conv, split.conv)


def test_conv_step_against_oracle(orc):
    M, C = 5, 3 * 64 * 128
    g = torch.Generator(device=DEV).manual_seed(7)
    x = torch.randn((M, C), generator=g, device=DEV).to(torch.bfloat16)
    w = (0.5 * torch.randn((C, 4), generator=g, device=DEV)).to(torch.bfloat16)
    cs = torch.randn((M, 3, C), generator=g, device=DEV).to(torch.bfloat16)
    cs_h = host(cs)
    y = torch.empty((M, C), dtype=torch.float32, device=DEV)
    out = torch.empty_like(cs)
    kda_conv_step(x, w, cs, out, y)
    torch.cuda.synchronize()
    for m in range(M):
        z, cs_ref = orc.conv_silu(host(x[m]), host(w), cs_h[m])
        assert np.array_equal(host(out[m]), cs_ref)
        assert rel_err(host(y[m]), z) <= 1e-6


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M", [4, 25, 33])
def test_recurrent_step_against_oracle(orc, state_dtype, M):
    """M = 33: 2112 heads, the launch that stores the state with agent scope."""
    H, D = 64, 128
    wl = kda_synth.custom("rec", M, H, D)
    S = kda_synth.initial_state(wl, 0, DEV, state_dtype)
    g = torch.Generator(device=DEV).manual_seed(9)
    qkv = torch.nn.functional.silu(torch.randn((M, 3, H * D), generator=g, device=DEV))
    inp = kda_synth.step_inputs(wl, 0, 0, DEV)
    o = torch.empty((M, H, D), dtype=torch.bfloat16, device=DEV)
    S0 = host(S)
    kda_recurrent_step(S, qkv, inp["alpha"], inp["beta"], wl.scale, o)
    torch.cuda.synchronize()
    S_ref, o_ref = orc.recurrent_step(S0, host(qkv), host(inp["alpha"]), host(inp["beta"]), wl.scale)
    assert rel_err(host(o), o_ref) <= TOL_O
    assert rel_err(host(S), S_ref) <= (1e-5 if state_dtype == "f32" else 4e-3)


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_alpha1_beta0_leaves_state_unchanged(state_dtype):
    wl = kda_synth.custom("ident", 4, 64, 128)
    lay = Layer(wl, 0, DEV, state_dtype)
    S0 = lay.state.clone()
    inp = kda_synth.step_inputs(wl, 0, 0, DEV)
    inp["alpha"].fill_(1.0)
    inp["beta"].zero_()
    lay.step(inp)
    torch.cuda.synchronize()
    assert torch.equal(lay.state, S0)


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_zero_input_is_pure_decay(state_dtype):
    wl = kda_synth.custom("zero", 2, 64, 128)
    lay = Layer(wl, 0, DEV, state_dtype)
    lay.conv.zero_()
    S0 = lay.state.clone()
    inp = kda_synth.step_inputs(wl, 0, 0, DEV)
    inp["x"].zero_()
    lay.step(inp)
    torch.cuda.synchronize()
    expect = (S0.float() * inp["alpha"][..., None]).to(S0.dtype)
    assert torch.equal(lay.state, expect)
    assert torch.count_nonzero(lay.o.float()) == 0


@pytest.mark.parametrize("pow2", [False, True])
def test_bf16_state_rounding_ties(pow2):
    """A pure decay by 1 + 2^-8 and 1 - 2^-8 leaves 8 bits below a bf16
    state's last place: round to nearest even decides every element, and a
    power-of-two state makes every one of the first kind an exact tie.  The
    expected state is rounded on the CPU."""
    wl = kda_synth.custom("ties", 2, 64, 128)
    lay = Layer(wl, 0, DEV, "bf16")
    if pow2:
        e = torch.randint(-20, 4, lay.state.shape, generator=torch.Generator().manual_seed(5))
        sign = torch.where(torch.rand(lay.state.shape, generator=torch.Generator().manual_seed(6)) < 0.5, -1.0, 1.0)
        lay.state.copy_((sign * torch.pow(2.0, e.double())).to(torch.bfloat16))
    lay.conv.zero_()
    S0 = lay.state.cpu()
    inp = kda_synth.step_inputs(wl, 0, 0, DEV)
    inp["x"].zero_()
    alpha = torch.full_like(inp["alpha"], 1.0 + 2.0 ** -8)
    alpha[..., 1::2] = 1.0 - 2.0 ** -8
    inp["alpha"].copy_(alpha)
    lay.step(inp)
    torch.cuda.synchronize()
    expect = (S0.float() * alpha.cpu()[..., None]).to(torch.bfloat16)
    assert torch.equal(lay.state.cpu(), expect)


def test_exact_recall_beta1(orc):
    """beta = 1 and q = k (same channels, same conv taps, scale 1): the read
    returns v up to the L2 norm's epsilon ("GLM-5.3 deep dive" 8.2.3)."""
    wl = kda_synth.custom("recall", 4, 64, 128)
    lay = Layer(wl, 0, DEV, "f32")
    HD = wl.H * wl.D
    lay.conv_w.view(3, HD, 4)[0] = lay.conv_w.view(3, HD, 4)[1]
    cv = lay.conv.view(wl.M, 3, 3, HD)
    cv[:, :, 0] = cv[:, :, 1]
    inp = kda_synth.step_inputs(wl, 0, 0, DEV)
    inp["x"][:, 0] = inp["x"][:, 1]
    inp["beta"].fill_(1.0)
    cs_before = host(lay.conv)
    kda_decode_step(lay.state, inp["x"], lay.conv_w, lay.conv, lay.conv, inp["alpha"], inp["beta"],
                    1.0, lay.o)
    torch.cuda.synchronize()
    v = np.stack([orc.conv_silu(host(inp["x"][m]).ravel(), host(lay.conv_w), cs_before[m])[0][2 * HD:]
                  for m in range(wl.M)]).reshape(wl.M, wl.H, wl.D)
    assert rel_err(host(lay.o), v) <= TOL_O


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_checkpoint_resume_bitwise(state_dtype):
    """8 steps in one go equal 4 steps, a copy of (state, conv state) to fresh
    buffers, and 4 more steps."""
    wl = kda_synth.custom("resume", 4, 64, 128, steps=8)
    a, oa = run(wl, state_dtype, 8)
    b = Layer(wl, 0, DEV, state_dtype)
    for t in range(4):
        b.step(kda_synth.step_inputs(wl, 0, t, DEV))
    b.state = b.state.clone()
    b.conv = b.conv.clone()
    for t in range(4, 8):
        b.step(kda_synth.step_inputs(wl, 0, t, DEV))
    torch.cuda.synchronize()
    assert torch.equal(a.state, b.state) and torch.equal(a.conv, b.conv)
    assert torch.equal(oa[-1], b.o)
