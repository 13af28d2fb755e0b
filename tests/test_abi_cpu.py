"""The C-ABI library loads, exports what include/kda.h declares, and rejects
bad arguments on the host before touching the GPU (no GPU needed).

Every call below is built to FAIL validation: the pointers are fake and are
never dereferenced.  No call here may pass validation, or it would launch.
"""
import math
import os
import re

import pytest
import torch

import hybrid_linear_attention_kda_amd as kda
from hybrid_linear_attention_kda_amd import kda as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

GAP = 1 << 30  # fake buffers 1 GiB apart never overlap at these sizes


def fake(i, misalign=0):
    return (i + 1) * GAP + misalign


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char \*)\s*(\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_version_and_status_strings(lib):
    assert kda.kda_version() == 10200
    for code in range(8):
        s = kda.kda_status_string(code)
        assert s and s != "unknown status"
    assert kda.kda_status_string(99) == "unknown status"


def decode(lib, M=1, H=64, D=128, sdt=0, ptrs=None, scale=0.125, nsplit=None, mis=None):
    p = [fake(i) for i in range(8)] if ptrs is None else list(ptrs)
    if mis is not None:
        p[mis] += 8
    state, x, w, cin, cout, a, b, o = p
    args = (M, H, D, sdt, state, x, w, cin, cout, a, b, scale, o, None)
    if nsplit is None:
        return lib.kda_decode_step(*args)
    return lib.kda_decode_step_split(*args, nsplit)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), binding.KDA_ERR_ARG),
    (dict(H=0), binding.KDA_ERR_SHAPE),
    (dict(D=48), binding.KDA_ERR_SHAPE),
    (dict(D=256), binding.KDA_ERR_SHAPE),
    (dict(sdt=2), binding.KDA_ERR_DTYPE),
    (dict(scale=math.nan), binding.KDA_ERR_ARG),
    (dict(scale=math.inf), binding.KDA_ERR_ARG),
    (dict(nsplit=3), binding.KDA_ERR_ARG),
    (dict(nsplit=0), binding.KDA_ERR_ARG),
    (dict(D=64, nsplit=2), binding.KDA_ERR_ARG),
])
def test_decode_argument_errors(lib, kw, code):
    assert decode(lib, **kw) == code


@pytest.mark.parametrize("which", range(8))
def test_decode_null_pointer(lib, which):
    p = [fake(i) for i in range(8)]
    p[which] = None
    assert decode(lib, ptrs=p) == binding.KDA_ERR_NULL


@pytest.mark.parametrize("which", range(8))
def test_decode_misaligned_pointer(lib, which):
    assert decode(lib, mis=which) == binding.KDA_ERR_ALIGN


def test_decode_empty_batch_touches_nothing(lib):
    assert decode(lib, M=0, ptrs=[None] * 8) == binding.KDA_OK


def test_decode_aliasing(lib):
    base = [fake(i) for i in range(8)]
    # state overlapping x
    p = list(base); p[1] = p[0] + 4096
    assert decode(lib, ptrs=p) == binding.KDA_ERR_ALIAS
    # o inside the state
    p = list(base); p[7] = p[0] + 1024
    assert decode(lib, ptrs=p) == binding.KDA_ERR_ALIAS
    # conv_out partially overlapping conv_in
    p = list(base); p[4] = p[3] + 16
    assert decode(lib, ptrs=p) == binding.KDA_ERR_ALIAS
    # conv_out overlapping alpha
    p = list(base); p[4] = p[5]
    assert decode(lib, ptrs=p) == binding.KDA_ERR_ALIAS
    # exact in-place conv state is allowed, but a split above 1 is not then
    p = list(base); p[4] = p[3]
    assert decode(lib, ptrs=p, nsplit=2) == binding.KDA_ERR_ARG


def test_conv_step_errors(lib):
    p = [fake(i) for i in range(5)]
    assert lib.kda_conv_step(-1, 64, *p, None) == binding.KDA_ERR_ARG
    assert lib.kda_conv_step(1, 12, *p, None) == binding.KDA_ERR_ARG
    assert lib.kda_conv_step(1, 0, *p, None) == binding.KDA_ERR_ARG
    assert lib.kda_conv_step(0, 64, None, None, None, None, None, None) == binding.KDA_OK
    for i in range(5):
        q = list(p); q[i] = None
        assert lib.kda_conv_step(1, 64, *q, None) == binding.KDA_ERR_NULL
        q = list(p); q[i] += 2
        assert lib.kda_conv_step(1, 64, *q, None) == binding.KDA_ERR_ALIGN
    q = list(p); q[4] = q[0]           # y over x
    assert lib.kda_conv_step(1, 64, *q, None) == binding.KDA_ERR_ALIAS
    q = list(p); q[3] = q[2] + 32      # conv_out partially over conv_in
    assert lib.kda_conv_step(1, 64, *q, None) == binding.KDA_ERR_ALIAS


def test_recurrent_step_errors(lib):
    p = [fake(i) for i in range(5)]   # state, qkv, alpha, beta, o
    def call(M=1, H=4, D=16, sdt=0, ptrs=p, scale=1.0):
        s, q, a, b, o = ptrs
        return lib.kda_recurrent_step(M, H, D, sdt, s, q, a, b, scale, o, None)
    assert call(M=-2) == binding.KDA_ERR_ARG
    assert call(D=8) == binding.KDA_ERR_SHAPE
    assert call(sdt=5) == binding.KDA_ERR_DTYPE
    assert call(scale=math.nan) == binding.KDA_ERR_ARG
    assert call(M=0, ptrs=[None] * 5) == binding.KDA_OK
    for i in range(5):
        q = list(p); q[i] = None
        assert call(ptrs=q) == binding.KDA_ERR_NULL
        q = list(p); q[i] += 4
        assert call(ptrs=q) == binding.KDA_ERR_ALIGN
    q = list(p); q[4] = q[0] + 64
    assert call(ptrs=q) == binding.KDA_ERR_ALIAS


# ----------------------------------------------- gated step and layer step --
# pointers: state, x, w, cin, cout, f, A_log, dt_bias, beta_logit, out[, out_gate, norm_w]
def gated(lib, M=1, H=64, D=128, sdt=0, ptrs=None, kind=0, lb=-5.0, scale=0.125, layer=False,
          norm_eps=1e-5, mis=None):
    n = 12 if layer else 10
    p = [fake(i) for i in range(n)] if ptrs is None else list(ptrs)
    if mis is not None:
        p[mis] += 8
    head = (M, H, D, sdt, *p[:9], kind, lb, scale)
    if layer:
        return lib.kda_decode_layer_step(*head, p[10], p[11], norm_eps, p[9], None)
    return lib.kda_decode_step_gated(*head, p[9], None)


@pytest.mark.parametrize("layer", [False, True], ids=["gated", "layer"])
@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), binding.KDA_ERR_ARG),
    (dict(D=48), binding.KDA_ERR_SHAPE),
    (dict(sdt=3), binding.KDA_ERR_DTYPE),
    (dict(scale=math.nan), binding.KDA_ERR_ARG),
    (dict(kind=2), binding.KDA_ERR_ARG),
    (dict(kind=-1), binding.KDA_ERR_ARG),
    (dict(kind=0, lb=0.0), binding.KDA_ERR_ARG),
    (dict(kind=0, lb=1.0), binding.KDA_ERR_ARG),
    (dict(kind=0, lb=math.nan), binding.KDA_ERR_ARG),
    (dict(kind=0, lb=-math.inf), binding.KDA_ERR_ARG),
])
def test_gated_argument_errors(lib, kw, code, layer):
    assert gated(lib, layer=layer, **kw) == code


@pytest.mark.parametrize("eps", [-1e-5, math.nan, math.inf])
def test_layer_norm_eps_errors(lib, eps):
    assert gated(lib, layer=True, norm_eps=eps) == binding.KDA_ERR_ARG


@pytest.mark.parametrize("layer,which", [(False, i) for i in range(10)] + [(True, i) for i in range(12)])
def test_gated_null_and_misaligned(lib, layer, which):
    n = 12 if layer else 10
    p = [fake(i) for i in range(n)]
    p[which] = None
    assert gated(lib, ptrs=p, layer=layer) == binding.KDA_ERR_NULL
    assert gated(lib, layer=layer, mis=which) == binding.KDA_ERR_ALIGN


def test_gated_empty_batch_touches_nothing(lib):
    assert gated(lib, M=0, ptrs=[None] * 10) == binding.KDA_OK
    assert gated(lib, M=0, ptrs=[None] * 12, layer=True) == binding.KDA_OK


def test_gated_aliasing(lib):
    base = [fake(i) for i in range(12)]
    for layer in (False, True):
        n = 12 if layer else 10
        p = list(base[:n]); p[9] = p[5]            # output over f_gate
        assert gated(lib, ptrs=p, layer=layer) == binding.KDA_ERR_ALIAS
        p = list(base[:n]); p[7] = p[0] + 256      # dt_bias inside the state
        assert gated(lib, ptrs=p, layer=layer) == binding.KDA_ERR_ALIAS
        p = list(base[:n]); p[8] = p[4] + 64       # beta_logit inside conv_out
        assert gated(lib, ptrs=p, layer=layer) == binding.KDA_ERR_ALIAS
    p = list(base); p[9] = p[10]                   # y over out_gate
    assert gated(lib, ptrs=p, layer=True) == binding.KDA_ERR_ALIAS
    p = list(base); p[11] = p[0] + 512             # norm weight inside the state
    assert gated(lib, ptrs=p, layer=True) == binding.KDA_ERR_ALIAS


# ------------------------------------------------------------ T tokens ----
def test_multi_errors(lib):
    p = [fake(i) for i in range(8)]   # state, x, w, cin, cout, alpha, beta, o

    def call(T=4, M=1, H=64, D=128, sdt=0, ptrs=p, scale=0.125):
        s, x, w, ci, co, a, b, o = ptrs
        return lib.kda_decode_multi(T, M, H, D, sdt, s, x, w, ci, co, a, b, scale, o, None)
    assert call(T=-1) == binding.KDA_ERR_ARG
    assert call(T=(1 << 30) + 1) == binding.KDA_ERR_ARG     # above KDA_MAX_TOKENS
    assert call(M=-1) == binding.KDA_ERR_ARG
    assert call(D=100) == binding.KDA_ERR_SHAPE
    assert call(sdt=9) == binding.KDA_ERR_DTYPE
    assert call(scale=math.inf) == binding.KDA_ERR_ARG
    assert call(T=0, ptrs=[None] * 8) == binding.KDA_OK
    assert call(M=0, ptrs=[None] * 8) == binding.KDA_OK
    for i in range(8):
        q = list(p); q[i] = None
        assert call(ptrs=q) == binding.KDA_ERR_NULL
        q = list(p); q[i] += 4
        assert call(ptrs=q) == binding.KDA_ERR_ALIGN
    q = list(p); q[7] = q[1] + 4096     # o over the tokens' x
    assert call(ptrs=q) == binding.KDA_ERR_ALIAS
    q = list(p); q[4] = q[5] + 16       # conv_out inside alpha
    assert call(ptrs=q) == binding.KDA_ERR_ALIAS
    # o of T tokens spans T times one token's output: alpha placed 64 KiB past
    # o is inside it at T = 64
    q = list(p); q[5] = q[7] + 64 * 1024
    assert call(T=64, ptrs=q) == binding.KDA_ERR_ALIAS


# ------------------------------------------------------------------ prefill --
def test_prefill_errors(lib):
    # state, x, w, cin, cout, f, A_log, dt_bias, beta_logit, o
    p = [fake(i) for i in range(10)]

    def call(L=32, M=1, H=64, D=128, sdt=0, ptrs=p, lb=-5.0, scale=0.125):
        s, x, w, ci, co, f, A, b, bl, o = ptrs
        return lib.kda_prefill_gated(L, M, H, D, sdt, s, x, w, ci, co, f, A, b, bl, lb, scale, o, None)
    assert call(L=-1) == binding.KDA_ERR_ARG
    assert call(L=(1 << 30) + 1) == binding.KDA_ERR_ARG     # above KDA_MAX_TOKENS
    assert call(D=64) == binding.KDA_ERR_SHAPE
    assert call(sdt=4) == binding.KDA_ERR_DTYPE
    for lb in (-5.5, 0.0, 0.5, math.nan, -math.inf):
        assert call(lb=lb) == binding.KDA_ERR_ARG, lb
    assert call(L=0, ptrs=[None] * 10) == binding.KDA_OK
    assert call(M=0, ptrs=[None] * 10) == binding.KDA_OK
    for i in range(10):
        q = list(p); q[i] = None
        assert call(ptrs=q) == binding.KDA_ERR_NULL
        q = list(p); q[i] += 4
        assert call(ptrs=q) == binding.KDA_ERR_ALIGN
    q = list(p); q[9] = q[5]            # o over f_gate
    assert call(ptrs=q) == binding.KDA_ERR_ALIAS
    q = list(p); q[0] = q[1] + 8192     # state inside x
    assert call(ptrs=q) == binding.KDA_ERR_ALIAS


def test_prefill_workspace_errors(lib):
    rec = 42496
    assert lib.kda_prefill_workspace_bytes(32, 2, 64, 128) == 2 * 2 * 64 * rec
    assert lib.kda_prefill_workspace_bytes(33, 1, 1, 128) == 3 * rec
    assert lib.kda_prefill_workspace_bytes(0, 1, 1, 128) == 0
    assert lib.kda_prefill_workspace_bytes(16, 1, 1, 64) == 0
    assert lib.kda_prefill_workspace_bytes(16, 0, 1, 128) == 0
    assert lib.kda_prefill_workspace_bytes(1 << 30, 1 << 12, 64, 128) == 0     # above 2^40
    p = [fake(i) for i in range(11)]     # ... as test_prefill_errors, then the workspace

    def call(L=32, M=1, H=64, D=128, sdt=0, ptrs=p, wsb=None, passes=0, lb=-5.0):
        s, x, w, ci, co, f, A, b, bl, o, ws = ptrs
        if wsb is None:
            wsb = lib.kda_prefill_workspace_bytes(L, M, H, D)
        return lib.kda_prefill_gated_ws(L, M, H, D, sdt, s, x, w, ci, co, f, A, b, bl, lb, 0.125, o, ws, wsb,
                                         passes, None)
    for ps in (-1, 3):
        assert call(passes=ps) == binding.KDA_ERR_ARG
    assert call(D=64) == binding.KDA_ERR_SHAPE
    assert call(lb=-6.0) == binding.KDA_ERR_ARG
    assert call(L=0, ptrs=[None] * 11) == binding.KDA_OK
    for ps in (0, 2):
        q = list(p); q[10] = None
        assert call(ptrs=q, passes=ps) == binding.KDA_ERR_NULL
        q = list(p); q[10] += 8
        assert call(ptrs=q, passes=ps) == binding.KDA_ERR_ALIGN
        # below one chunk's records for every head
        assert call(wsb=64 * rec - 16, passes=ps) == binding.KDA_ERR_ARG
        # bf16 state with a partial workspace also needs the f32 stage
        assert call(sdt=1, wsb=64 * rec, passes=ps) == binding.KDA_ERR_ARG
        q = list(p); q[10] = q[1] + 4096    # workspace inside x
        assert call(ptrs=q, passes=ps) == binding.KDA_ERR_ALIAS
        q = list(p); q[10] = q[0] - 4096    # workspace running into the state
        assert call(ptrs=q, passes=ps) == binding.KDA_ERR_ALIAS


def test_prefill_noalloc_errors(lib):
    """The allocation-free prefill validates like kda_prefill_gated before
    any HIP call (fake pointers, never dereferenced)."""
    p = [fake(i) for i in range(10)]

    def call(L=32, M=1, H=64, D=128, sdt=0, ptrs=p, lb=-5.0, scale=0.125):
        s, x, w, ci, co, f, A, b, bl, o = ptrs
        return lib.kda_prefill_gated_noalloc(L, M, H, D, sdt, s, x, w, ci, co, f, A, b, bl, lb, scale, o, None)
    assert call(L=-1) == binding.KDA_ERR_ARG
    assert call(D=64) == binding.KDA_ERR_SHAPE
    assert call(sdt=2) == binding.KDA_ERR_DTYPE
    assert call(lb=0.0) == binding.KDA_ERR_ARG
    assert call(scale=math.inf) == binding.KDA_ERR_ARG
    assert call(L=0, ptrs=[None] * 10) == binding.KDA_OK
    for i in range(10):
        q = list(p); q[i] = None
        assert call(ptrs=q) == binding.KDA_ERR_NULL
        q = list(p); q[i] += 4
        assert call(ptrs=q) == binding.KDA_ERR_ALIGN
    q = list(p); q[9] = q[1]            # o over x
    assert call(ptrs=q) == binding.KDA_ERR_ALIAS


def test_binding_rejects_host_tensors():
    M, H, D = 1, 2, 16
    st = torch.zeros(M, H, D, D)
    with pytest.raises(ValueError):
        kda.kda_decode_step(st, None, None, None, None, None, None, 1.0, None)
    with pytest.raises(ValueError):
        kda.kda_recurrent_step(st, None, None, None, 1.0, None)
    with pytest.raises(ValueError):
        kda.kda_conv_step(torch.zeros(1, 8, dtype=torch.bfloat16), None, None, None, None)


# ------------------------------------------------------- measurement probes --
def test_probe_library_exports_and_rejects_bad_arguments():
    """libkda_probe.so exports what include/kda_probe.h declares; every call
    here fails host validation (fake pointers, never dereferenced)."""
    from hybrid_linear_attention_kda_amd import probe
    text = open(os.path.join(ROOT, "include", "kda_probe.h")).read()
    names = sorted(set(re.findall(r"^int\s*(\w+)\(", text, re.M)))
    assert set(names) == set(probe.EXPORTS)
    plib = probe.load()
    for n in names:
        assert hasattr(plib, n), f"libkda_probe.so does not export {n}"
    assert plib.kda_probe_rmw(None, 8192, 1.0, None) == 1
    assert plib.kda_probe_rmw(fake(0, 8), 8192, 1.0, None) == 4
    assert plib.kda_probe_rmw(fake(0), 0, 1.0, None) == 6
    assert plib.kda_probe_rmw(fake(0), 8192 + 16, 1.0, None) == 6
    assert plib.kda_probe_copy(fake(0), None, 8192, None) == 1
    assert plib.kda_probe_copy(fake(0), fake(0, 8), 8192, None) == 4
    assert plib.kda_probe_copy(fake(0), fake(0) + 4096, 8192, None) == 5
    assert plib.kda_probe_copy(fake(0), fake(1), 100, None) == 6
    st = plib.kda_probe_stream
    assert st(4, 512, 1, 0, fake(0), fake(0), 8192, 1.0, None) == 6          # unknown kind
    assert st(0, 512, 1, 0, None, None, 8192, 1.0, None) == 1
    assert st(1, 512, 1, 0, None, None, 8192, 1.0, None) == 1                 # read only needs src
    assert st(2, 512, 1, 0, fake(0), None, 8192, 1.0, None) == 1              # write only needs dst
    assert st(0, 512, 1, 0, fake(0, 8), fake(0, 8), 8192, 1.0, None) == 4
    assert st(0, 512, 1, 0, fake(0), fake(1), 8192, 1.0, None) == 5           # in place: dst == src
    assert st(3, 512, 1, 0, fake(0), fake(0) + 4096, 8192, 1.0, None) == 5    # copy: no overlap
    assert st(0, 384, 1, 0, fake(0), fake(0), 8192, 1.0, None) == 6           # threads
    assert st(0, 512, 3, 0, fake(0), fake(0), 8192, 1.0, None) == 6           # chunks per lane
    assert st(0, 1024, 4, 0, fake(0), fake(0), 32768, 1.0, None) == 6         # not a whole tile
    assert st(0, 512, 1, 0, fake(0), fake(0), 0, 1.0, None) == 6
