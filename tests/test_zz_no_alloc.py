"""kda_prefill_gated_noalloc (the two-pass prefill through the library's own
device scratch array, for callers that cannot allocate) through the C ABI,
against kda_prefill_gated_ws with a caller workspace large enough for one
segment: states, outputs and conv states bit-identical (the segmented and
one-segment two-pass forms perform the same operations in the same order).
Two calls in a row share the scratch array, the second with a smaller
input; a third shape takes the one-pass route, which uses no scratch."""
import ctypes

import pytest
import torch

import kda_synth
from hybrid_linear_attention_kda_amd import kda

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
vp = ctypes.c_void_p


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()


def inputs(M, H, L, sdt, seed):
    wl = kda_synth.custom(f"noalloc_{M}_{H}_{L}", M, H, 128, steps=L, seed=seed)
    li = kda_synth.layer_inputs(wl, 0, DEV, sdt)
    gp = kda_synth.gate_params(wl, 0, DEV)
    seq = kda_synth.sequence_inputs(wl, 0, L, DEV)
    return wl, li, gp, seq


def run(lib, which, M, H, L, sdt, wl, li, gp, seq, inplace):
    S = li["state"].clone()
    cin = li["conv_state"].clone()
    cout = cin if inplace else torch.empty_like(cin)
    o = torch.empty((M, L, H, 128), dtype=torch.bfloat16, device=DEV)
    code = kda.KDA_STATE_F32 if sdt == "f32" else kda.KDA_STATE_BF16
    head = (L, M, H, 128, code, vp(S.data_ptr()), vp(seq["x"].data_ptr()), vp(li["conv_w"].data_ptr()),
            vp(cin.data_ptr()), vp(cout.data_ptr()), vp(seq["f"].data_ptr()), vp(gp["A_log"].data_ptr()),
            vp(gp["dt_bias"].data_ptr()), vp(seq["beta_logit"].data_ptr()), ctypes.c_float(-5.0),
            ctypes.c_float(wl.scale), vp(o.data_ptr()))
    stream = vp(torch.cuda.current_stream().cuda_stream)
    if which == "noalloc":
        rc = lib.kda_prefill_gated_noalloc(*head, stream)
    else:
        wsb = lib.kda_prefill_workspace_bytes(L, M, H, 128)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        rc = lib.kda_prefill_gated_ws(*head, vp(ws.data_ptr()), wsb, 0, stream)
    assert rc == 0, kda.status_string(rc)
    torch.cuda.synchronize()
    return S, o, cout


@pytest.mark.parametrize("M,H,L,sdt,inplace", [
    (1, 64, 1100, "f32", False),    # several segments of the 64 MiB array
    (1, 16, 200, "bf16", True),     # then a smaller call on the same array
    (4, 64, 40, "f32", False),      # 2 M H above the CU count: one pass, no scratch
])
def test_noalloc_matches_workspace_entry(M, H, L, sdt, inplace):
    lib = kda.load()
    wl, li, gp, seq = inputs(M, H, L, sdt, seed=21)
    ref = run(lib, "ws", M, H, L, sdt, wl, li, gp, seq, inplace)
    got = run(lib, "noalloc", M, H, L, sdt, wl, li, gp, seq, inplace)
    for name, a, b in zip(("state", "outputs", "conv state"), ref, got):
        assert torch.equal(a, b), name
    print(f"noalloc ({M},{H},L={L}) {sdt}: bit-identical to the workspace entry point", flush=True)
