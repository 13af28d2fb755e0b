#!/usr/bin/env python3
"""Benchmark of the KDA decode step on one MI355X.

One "step" is one token through all 34 KDA layers of GLM-5.3-Flash: 34
launches of the fused decode kernel, each over M streams x 64 heads x
128 x 128 state, every layer with its own state (so the state is read from
HBM, not from the 256 MiB Infinity Cache).  Inputs are synthetic
(``kda_synth``), resident in HBM before timing starts: the headline draws a
fresh input set (q/k/v, alpha, beta) for every timed step; the secondary
lines rotate up to 8 sets.

Headline: M = 32 streams, FP32 state.  Also measured (``secondary``): M = 8
with FP32 and BF16 state, M = 128 with BF16 state, M = 1, the gated and
layer steps, T = 8 tokens per call, and the chunked prefill (tokens/s and
FP32-equivalent TFLOP/s for M streams x L tokens of one layer).

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints ONE JSON line.  ``value`` is state GB/s = 2 * M * H * D^2 * bytes per
layer (state read + written) over the measured time.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "decode_kernel_traffic.json")
# the sources the decode kernel is compiled from (the stored counter traffic
# is reported only while they are unchanged)
KERNEL_SOURCES = [os.path.join(ROOT, "hybrid_linear_attention_kda_amd", "csrc", n)
                  for n in ("kda_kernels.hip", "kda_device.h")]
METRIC = "KDA decode state GB/s + ms/layer at M=8,32 (FP32/BF16 state), % HBM peak"

# algorithmic bytes besides the state, (per stream, per layer): the plain
# step reads x 49,152, reads and writes the conv state 294,912, reads alpha
# 32,768 and beta 256 and writes o 16,384 per stream; conv weights 196,608
# per layer.  The gated step takes the raw gate instead of alpha and beta: x + conv state
# + f 16,384 + beta logit 128 + o 16,384 per stream; dt_bias 32,768 and
# A_log 256 per layer.  The layer step adds the output gate (16,384 per
# stream) and the norm weight (512 per layer); y replaces o.
SIDE_BYTES = {"plain": (393_472, 196_608), "gated": (376_960, 196_608 + 32_768 + 256),
              "layer": (393_344, 196_608 + 32_768 + 256 + 512)}
# T tokens per call: per stream and token x 49,152 + alpha 32,768 + beta 256
# + o 16,384; the conv state 294,912 once per call
MULTI_TOKEN_BYTES, MULTI_CALL_BYTES = 98_560, 294_912
MULTI_T = 8
CONV_W_BYTES = 196_608
# chunked prefill (16-token chunks, D = 128), per (chunk, head), as the chunk
# form is computed: the intra-chunk products A and P 2 x 2 C^2 D, the
# triangular solves for W and U by substitution 2 x 2 (C (C - 1) / 2) D, the
# state products W S and (Gamma Q) S 2 x 2 C D^2, P Delta 2 C^2 D, the state
# update 2 C D^2 -> 1,830,912 flops (FP32-equivalent: each is computed to
# FP32 accuracy)
PREFILL_FLOPS_PER_CHUNK_HEAD = 1_830_912
# bf16 matrix-core flops the kernels issue for the three state products,
# per (chunk, head): W S and the update from three-way splits with six piece
# products each, (Gamma Q) S with three -> (6 + 3 + 6) x 2 C D^2
PREFILL_BF16_MFMA_FLOPS_PER_CHUNK_HEAD = 15 * 2 * 16 * 128 * 128
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix
PREFILL_CHUNK = 16
# per stream and token: x 49,152 + f 16,384 + beta logit 128 + o 16,384 read or
# written; per stream the conv state 294,912; per layer conv w, dt_bias, A_log
PREFILL_TOKEN_BYTES, PREFILL_STREAM_BYTES = 82_048, 294_912
PREFILL_LAYER_BYTES = 196_608 + 32_768 + 256
MFMA_F32_PEAK_TFLOPS = 157.3     # MI355X dense FP32 matrix
# (streams, tokens per stream, state dtype) of the prefill lines; the last two are
# the T-token shapes of kda_decode_multi, for the chunked path
PREFILL_SHAPES = ((8, 2048, "f32"), (1, 8192, "f32"), (2, 4096, "f32"), (1, 4096, "bf16"), (32, 1024, "bf16"),
                  (32, 8, "f32"), (32, 16, "f32"))
PREFILL_WARM_S = 0.1              # least time of back-to-back warm-up launches per prefill line


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Model:
    """34 layers of device buffers plus pre-marshalled C-ABI arguments."""

    def __init__(self, wl, state_dtype, n_inputs, device="cuda:0", mode="plain", T=1):
        import torch

        import kda_synth
        from hybrid_linear_attention_kda_amd import kda

        self.wl, self.state_dtype = wl, state_dtype
        self.lib = kda.load()
        M, H, D = wl.M, wl.H, wl.D
        self.layers = []
        for layer in range(wl.layers):
            li = kda_synth.layer_inputs(wl, layer, device, state_dtype)
            o = torch.empty((M, H, D), dtype=torch.bfloat16, device=device)
            if mode == "multi":
                # input set t = tokens [t*T, (t+1)*T), stacked on a token axis
                ins = []
                for t in range(n_inputs):
                    toks = [kda_synth.step_inputs(wl, layer, t * T + j, device) for j in range(T)]
                    ins.append({k: torch.stack([tk[k] for tk in toks], 1).contiguous()
                                for k in ("x", "alpha", "beta")})
                o = torch.empty((M, T, H, D), dtype=torch.bfloat16, device=device)
            else:
                ins = [kda_synth.step_inputs(wl, layer, t, device) for t in range(n_inputs)]
            entry = {"state": li["state"], "conv_w": li["conv_w"], "conv": li["conv_state"],
                     "o": o, "inputs": ins}
            if mode != "plain":
                entry["gp"] = kda_synth.gate_params(wl, layer, device)
                entry["gi"] = [kda_synth.gate_inputs(wl, layer, t, device) for t in range(n_inputs)]
            self.layers.append(entry)
        torch.cuda.synchronize()
        sdt = kda.KDA_STATE_F32 if state_dtype == "f32" else kda.KDA_STATE_BF16
        self.n_inputs = n_inputs
        self.mode, self.T = mode, T
        self.args = []   # [input set][layer] -> tuple of C arguments (stream last)
        vp = ctypes.c_void_p
        for t in range(n_inputs):
            row = []
            for L in self.layers:
                inp = L["inputs"][t]
                head = (M, H, D, sdt, vp(L["state"].data_ptr()), vp(inp["x"].data_ptr()),
                        vp(L["conv_w"].data_ptr()), vp(L["conv"].data_ptr()), vp(L["conv"].data_ptr()))
                if mode in ("plain", "multi"):
                    args = head + (vp(inp["alpha"].data_ptr()), vp(inp["beta"].data_ptr()),
                                   ctypes.c_float(wl.scale), vp(L["o"].data_ptr()))
                    row.append(args if mode == "plain" else (T,) + args)
                    continue
                gi, gp = L["gi"][t], L["gp"]
                gated = head + (vp(gi["f"].data_ptr()), vp(gp["A_log"].data_ptr()),
                                vp(gp["dt_bias"].data_ptr()), vp(gi["beta_logit"].data_ptr()),
                                kda.KDA_GATE_BOUNDED, ctypes.c_float(-5.0), ctypes.c_float(wl.scale))
                if mode == "gated":
                    row.append(gated + (vp(L["o"].data_ptr()),))
                else:
                    row.append(gated + (vp(gi["out_gate"].data_ptr()), vp(gp["norm_w"].data_ptr()),
                                        ctypes.c_float(1e-5), vp(L["o"].data_ptr())))
            self.args.append(row)

    def state_bytes_per_layer(self):
        return self.wl.state_bytes(self.state_dtype)

    def alg_bytes_per_launch(self):
        if self.mode == "multi":
            return (self.state_bytes_per_layer() * 2 + CONV_W_BYTES
                    + self.wl.M * (self.T * MULTI_TOKEN_BYTES + MULTI_CALL_BYTES))
        per_stream, per_layer = SIDE_BYTES[self.mode]
        return self.state_bytes_per_layer() * 2 + self.wl.M * per_stream + per_layer

    def step(self, t, stream_ptr):
        fn = {"plain": self.lib.kda_decode_step, "gated": self.lib.kda_decode_step_gated,
              "layer": self.lib.kda_decode_layer_step, "multi": self.lib.kda_decode_multi}[self.mode]
        s = ctypes.c_void_p(stream_ptr)
        for a in self.args[t % self.n_inputs]:
            rc = fn(*a, s)
            if rc:
                raise RuntimeError(f"{self.mode} decode step returned {rc}")


def time_model(model, steps, warmup, use_graph, per_step_events=False, hooks=None):
    """Return (seconds for `steps` steps, mode, per-step seconds or None).
    With per_step_events an event is recorded after every step (for the
    median and best step); that marker costs time, so the pass that gives
    the mean runs without it.  Timed step k takes input set k % n_inputs.
    `hooks` = (before, after): called (outside the timed region, after a
    device synchronisation) right before the first and right after the last
    timed step."""
    import torch
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        sp = stream.cuda_stream
        for w in range(warmup):
            model.step(w, sp)
        stream.synchronize()
        graphs = None
        if use_graph:
            graphs = []
            for t in range(model.n_inputs):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    model.step(t, torch.cuda.current_stream().cuda_stream)
                graphs.append(g)
            for g in graphs:           # one untimed replay of each
                g.replay()
            stream.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if per_step_events else None
        torch.cuda.synchronize()
        if hooks is not None:
            hooks[0]()
            torch.cuda.synchronize()
        start.record(stream)
        for k in range(steps):
            if graphs is not None:
                graphs[k % len(graphs)].replay()
            else:
                model.step(k, sp)
            if marks is not None:
                marks[k].record(stream)
        end.record(stream)
        end.synchronize()
        torch.cuda.synchronize()
        if hooks is not None:
            hooks[1]()
            torch.cuda.synchronize()
    per_step = None
    if marks is not None:
        per_step = [(marks[k - 1] if k else start).elapsed_time(marks[k]) / 1e3 for k in range(steps)]
    return start.elapsed_time(end) / 1e3, ("hipGraph" if use_graph else "eager"), per_step


# sampled units of the oracle check after the timed headline pass: (stream,
# head) pairs spread over the batch, in three layers
PARITY_LAYERS = (0, 17, 33)
PARITY_UNITS = ((0, 0), (9, 63), (21, 17), (31, 42))
TOL_STATE_F32, TOL_O = 1e-5, 4e-3


def _snapshot(model):
    return [(L["state"].clone(), L["conv"].clone(), L["o"].clone()) for L in model.layers]


def _f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def _rel(gpu, ref):
    import numpy as np
    den = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(gpu - ref)))
    return err / den if den > 0 else err


def timed_pass_parity(model, start, final, steps):
    """The timed pass against a separate, untimed correctness pass.

    From the states the timed pass started from (`start`), the same `steps`
    steps run again eagerly; the 34 layers' final states, conv states and
    outputs must equal the timed pass's (`final`) bit for bit (the kernels
    have no atomics or order-dependent sums).  Then sampled (stream, head)
    units of three layers go through the CPU oracle over the same steps from
    the same starting states, free-running, and are compared with the timed
    pass's final state (FP32 storage: 1e-5) and last output (4e-3), relative
    to the largest reference magnitude over the layer's sampled units (the
    state-tile page's *Correctness* metric)."""
    import numpy as np
    import torch

    import oracle
    wl = model.wl
    assert model.state_dtype == "f32" and model.mode == "plain"
    for L, (st, cv, _) in zip(model.layers, start):
        L["state"].copy_(st)
        L["conv"].copy_(cv)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for k in range(steps):
            model.step(k, stream.cuda_stream)
    stream.synchronize()
    bitwise = all(torch.equal(L["state"], f[0]) and torch.equal(L["conv"], f[1]) and torch.equal(L["o"], f[2])
                  for L, f in zip(model.layers, final))
    orc = oracle.get()
    H, D = wl.H, wl.D
    worst_s = worst_o = 0.0
    for li in PARITY_LAYERS:
        Lr = model.layers[li]
        w = _f64(Lr["conv_w"]).reshape(3, H, D, 4)
        cs0 = _f64(start[li][1])
        S0 = start[li][0]
        refs, gpus = [], []
        for m, h in PARITY_UNITS:
            S = _f64(S0[m, h]).reshape(1, 1, D, D)
            cs = cs0[m].reshape(3, 3, H, D)[:, :, h].reshape(1, 3, 3 * D)
            wu = w[:, h].reshape(3 * D, 4)
            for k in range(steps):
                inp = Lr["inputs"][k % model.n_inputs]
                x = _f64(inp["x"][m].reshape(3, H, D)[:, h]).reshape(1, 3, D)
                a = _f64(inp["alpha"][m, h]).reshape(1, 1, D)
                b = _f64(inp["beta"][m, h]).reshape(1, 1)
                S, cs, o = orc.decode_step(S, x, wu, cs, a, b, wl.scale)
            refs.append((S.reshape(D, D), o.reshape(D)))
            gpus.append((_f64(final[li][0][m, h]), _f64(final[li][2][m, h])))
        worst_s = max(worst_s, _rel(np.stack([g[0] for g in gpus]), np.stack([r[0] for r in refs])))
        worst_o = max(worst_o, _rel(np.stack([g[1] for g in gpus]), np.stack([r[1] for r in refs])))
    ok = bitwise and worst_s <= TOL_STATE_F32 and worst_o <= TOL_O
    return {"pass": ok, "bitwise_equal_to_untimed_pass": bitwise,
            "oracle_state_rel_err": worst_s, "oracle_o_rel_err": worst_o,
            "tolerance": {"state_f32": TOL_STATE_F32, "o": TOL_O},
            "sampled": f"layers {list(PARITY_LAYERS)} x (stream, head) {[list(u) for u in PARITY_UNITS]}, "
                       f"{steps} consecutive steps free-running from the timed pass's starting states"}


def measure(wl, state_dtype, steps, warmup, n_inputs, mode="plain", T=1, check=False):
    import torch
    model = Model(wl, state_dtype, n_inputs, mode=mode, T=T)
    res, snaps = {}, {}
    for use_graph in (False, True):
        box = {}
        hooks = ((lambda: box.__setitem__("start", _snapshot(model))),
                 (lambda: box.__setitem__("final", _snapshot(model)))) if check else None
        sec, mname, _ = time_model(model, steps, warmup, use_graph, hooks=hooks)
        snaps[mname] = box
        _, _, per_step = time_model(model, max(10, steps // 4), 1, use_graph, per_step_events=True)
        launches = steps * wl.layers
        srt = sorted(per_step)
        res[mname] = {
            "ms_per_step": sec * 1e3 / steps,
            "ms_per_layer": sec * 1e3 / launches,
            "ms_per_layer_median_step": srt[len(srt) // 2] * 1e3 / wl.layers,
            "ms_per_layer_best_step": srt[0] * 1e3 / wl.layers,
            "state_GBps": 2 * model.state_bytes_per_layer() * launches / sec / 1e9,
            "alg_GBps": model.alg_bytes_per_launch() * launches / sec / 1e9,
        }
    best = max(res, key=lambda m: res[m]["state_GBps"])
    out = dict(res[best])
    out["launch"] = best
    out["modes"] = res
    out["alg_bytes_per_launch"] = model.alg_bytes_per_launch()
    out["state_bytes_per_launch"] = 2 * model.state_bytes_per_layer()
    if check:
        # the reported (faster) launch mode's timed pass
        snaps = {best: snaps[best]}
        torch.cuda.empty_cache()
        out["timed_pass_parity"] = timed_pass_parity(model, snaps[best]["start"], snaps[best]["final"], steps)
        out["timed_pass_parity"]["launch"] = best
    del model, snaps
    torch.cuda.empty_cache()
    return out


def measure_prefill(M, L, state_dtype, steps, warmup, H=64, D=128):
    """kda_prefill_gated_ws over M streams x L tokens of one layer, launched
    `steps` times on the same buffers (state and conv state carried along):
    while 2 M H is at most the CU count the library chooses (passes = 0: two
    passes) over a one-segment workspace allocated before timing, else the
    one-pass form is asked for (passes = 1, no workspace)."""
    import torch

    import kda_synth
    from hybrid_linear_attention_kda_amd import kda
    lib = kda.load()
    wl = kda_synth.custom(f"prefill_m{M}_l{L}", M, H, D, steps=L, seed=7)
    li = kda_synth.layer_inputs(wl, 0, "cuda:0", state_dtype)
    gp = kda_synth.gate_params(wl, 0, "cuda:0")
    seq = kda_synth.sequence_inputs(wl, 0, L, "cuda:0")
    o = torch.empty((M, L, H, D), dtype=torch.bfloat16, device="cuda:0")
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    two = 2 * M * H <= ncu
    wsb = lib.kda_prefill_workspace_bytes(L, M, H, D) if two else 16
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    vp = ctypes.c_void_p
    sdt = kda.KDA_STATE_F32 if state_dtype == "f32" else kda.KDA_STATE_BF16
    stream = torch.cuda.Stream()
    # the conv state alternates between two buffers (conv_in != conv_out)
    cs = (li["conv_state"], li["conv_state"].clone())
    args = [(L, M, H, D, sdt, vp(li["state"].data_ptr()), vp(seq["x"].data_ptr()),
             vp(li["conv_w"].data_ptr()), vp(cs[i].data_ptr()), vp(cs[1 - i].data_ptr()),
             vp(seq["f"].data_ptr()), vp(gp["A_log"].data_ptr()), vp(gp["dt_bias"].data_ptr()),
             vp(seq["beta_logit"].data_ptr()), ctypes.c_float(-5.0), ctypes.c_float(wl.scale),
             vp(o.data_ptr()), vp(ws.data_ptr()), wsb, 0 if two else 1, vp(stream.cuda_stream)) for i in (0, 1)]
    calls = [0]

    def launch():
        rc = lib.kda_prefill_gated_ws(*args[calls[0] & 1])
        calls[0] += 1
        if rc:
            raise RuntimeError(f"kda_prefill_gated_ws returned {rc}")

    with torch.cuda.stream(stream):
        # at least `warmup` launches and PREFILL_WARM_S seconds of back-to-back
        # launches: the compute-bound chunk loop runs up to 10% slower until
        # the clock has settled under load (2 launches: 1.41-1.50 ms at
        # 8 x 2048, 20 or more: 1.35 ms; the memory-bound decode is the same
        # after 10 or 300 warm-up steps)
        t_warm = time.perf_counter()
        n_warm = 0
        while n_warm < warmup or time.perf_counter() - t_warm < PREFILL_WARM_S:
            launch()
            n_warm += 1
            if n_warm % 4 == 0:
                stream.synchronize()
        stream.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(steps):
            launch()
        e.record(stream)
        e.synchronize()
    sec = s.elapsed_time(e) / 1e3 / steps
    # per token (a ragged last chunk counts its tokens, not the padded 16)
    flops = PREFILL_FLOPS_PER_CHUNK_HEAD * M * H * L // PREFILL_CHUNK
    bf16_flops = PREFILL_BF16_MFMA_FLOPS_PER_CHUNK_HEAD * M * H * ((L + PREFILL_CHUNK - 1) // PREFILL_CHUNK)
    nbytes = (M * (L * PREFILL_TOKEN_BYTES + PREFILL_STREAM_BYTES) + PREFILL_LAYER_BYTES
              + 2 * wl.state_bytes(state_dtype))
    if two:
        nbytes += 2 * wsb          # pass 1 writes every chunk's record, pass 2 reads it
    del li, gp, seq, o, cs, ws
    torch.cuda.empty_cache()
    return {"workload": f"prefill_m{M}_l{L}", "M": M, "L": L, "H": H, "D": D,
            "state_dtype": state_dtype, "entry_point": "kda_prefill_gated_ws",
            "form": "two-pass" if two else "one-pass", "workspace_bytes": wsb if two else 0, "launch": "eager",
            "ms_per_layer": sec * 1e3, "tokens_per_s_per_layer": M * L / sec,
            "us_per_token_layer": sec * 1e6 / (M * L),
            "roofline": {"bound": "alu", "achieved": flops / sec / 1e12, "peak": MFMA_F32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / sec / 1e12 / MFMA_F32_PEAK_TFLOPS,
                         "achieved_is": "FP32-equivalent flops of the chunk form as computed (W and U by "
                                        "substitution) over time, against MI355X's FP32 peak",
                         "limiter": ("pass 2's per-chunk dependency chain (one chunk at a time per head)"
                                     if two else "VALU issue and LDS/barrier latency (counters in profiles/)"),
                         "bf16_mfma_TFLOPs_executed": bf16_flops / sec / 1e12,
                         "bf16_mfma_frac": bf16_flops / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                         "flops_per_launch": flops, "alg_bytes_per_launch": nbytes,
                         "alg_GBps": nbytes / sec / 1e9}}


def stream_ceiling(chunk_bytes, layers, steps, warmup=3):
    """The probe kernels (``libkda_probe.so``) over `layers` distinct chunks of
    `chunk_bytes` each, one launch per chunk as the decode step launches one
    per layer: the achievable rate of the decode's access contract.
    Returns {"rmw": GB/s, "copy": GB/s, "rmw_avg_launch_us": ...}; GB/s
    counts bytes read + written."""
    import torch

    from hybrid_linear_attention_kda_amd import probe
    plib = probe.load()
    n = chunk_bytes // 4
    buf = torch.ones(layers * n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(buf)
    stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    chunks = [(buf.data_ptr() + i * chunk_bytes, dst.data_ptr() + i * chunk_bytes) for i in range(layers)]

    def rmw():
        for a, _ in chunks:
            assert plib.kda_probe_rmw(ctypes.c_void_p(a), chunk_bytes, 1.0, sp) == 0

    def copy():
        for a, b in chunks:
            assert plib.kda_probe_copy(ctypes.c_void_p(a), ctypes.c_void_p(b), chunk_bytes, sp) == 0

    out = {}
    for name, fn in (("rmw", rmw), ("copy", copy)):
        for _ in range(warmup):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(steps):
            fn()
        e.record(stream)
        e.synchronize()
        sec = s.elapsed_time(e) / 1e3
        out[name] = 2 * chunk_bytes * layers * steps / sec / 1e9
        out[name + "_avg_launch_us"] = sec / (layers * steps) * 1e6
    del buf, dst
    torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, budget_s=12.0):
    """The CPU oracle (double precision, OpenMP over (stream, head) units) on a
    bounded sample of the same workload: layer after layer, each through all
    of the workload's consecutive steps, until about `budget_s` seconds of
    oracle time are spent.  Inputs are drawn on the host (same recipe) and
    converted outside the timed region; the timer brackets only the C
    routine, which updates a preallocated float64 state in place (the conv
    state alternates between two preallocated buffers)."""
    import ctypes as ct

    import numpy as np
    import torch

    import kda_synth
    import oracle
    orc = oracle.get()
    P = ct.POINTER(ct.c_double)
    ptr = lambda a: a.ctypes.data_as(P)  # noqa: E731
    h = lambda t: np.ascontiguousarray(t.to(torch.float64).numpy())  # noqa: E731
    M, H, D = wl.M, wl.H, wl.D
    layers, launches, elapsed = 0, 0, 0.0
    o = np.empty((M, H, D))
    while elapsed < budget_s and layers < wl.layers:
        li = kda_synth.layer_inputs(wl, layers, "cpu", "f32")
        S, w = h(li["state"]), h(li["conv_w"])
        cs = [h(li["conv_state"]), np.empty((M, 3, 3 * H * D))]
        for t in range(wl.steps):
            inp = kda_synth.step_inputs(wl, layers, t, "cpu")
            x, a, b = h(inp["x"]), h(inp["alpha"]), h(inp["beta"])
            t0 = time.perf_counter()
            rc = orc.lib.kda_oracle_decode_step(M, H, D, ptr(S), ptr(x), ptr(w), ptr(cs[0]), ptr(cs[1]), ptr(a),
                                                ptr(b), float(wl.scale), float(oracle.L2NORM_EPS), ptr(o))
            elapsed += time.perf_counter() - t0
            if rc != 0:
                raise RuntimeError(f"kda_oracle_decode_step failed ({rc})")
            cs.reverse()
            launches += 1
        layers += 1
    state_bytes = 2 * wl.state_bytes("f32") * launches
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": state_bytes / elapsed / 1e9,
        "unit": "GB/s",
        "cores": orc.max_threads(),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"{layers} of {wl.layers} layers x {wl.steps} steps of the same workload "
                  f"(M={wl.M}, 64x128x128; GB/s counts the FP32 state bytes the GPU moves), "
                  f"{elapsed:.1f} s of oracle time (the C routine only, state updated in place), "
                  f"{elapsed / launches * 1e3:.1f} ms per layer-step",
    }


def _counter_means(run_dir, counter):
    """{kernel name: (mean counter value, mean grid size, dispatches)} from a
    rocprofv3 --pmc CSV directory (values averaged over dispatches)."""
    import csv
    import glob
    import collections
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {run_dir}")
    acc = collections.defaultdict(lambda: [0.0, 0.0, 0])
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                a = acc[row["Kernel_Name"]]
                a[0] += float(row["Counter_Value"])
                a[1] += float(row["Grid_Size"])
                a[2] += 1
    return {k: (v[0] / v[2], v[1] / v[2], v[2]) for k, v in acc.items()}


def traffic_from_counters(fetch_dir, write_dir, out=TRAFFIC_FILE):
    """HBM bytes per headline decode launch from FETCH_SIZE and WRITE_SIZE,
    each scaled by what the same counter reads for the probe's in-place rmw
    (grid size x 16 bytes read and the same written), and stored (in `out`)
    with the kernel source's hash so that a later kernel change voids it."""
    decode_key = "decode_kernel<float, 128, 1, 16, 4"
    fetch, write = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")

    def pick(table, key):
        hits = [(k, v) for k, v in table.items() if key in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {key!r}, found {[k for k, _ in hits]}")
        return hits[0][1]

    f_dec, f_probe = pick(fetch, decode_key), pick(fetch, "rmw_kernel")
    w_dec, w_probe = pick(write, decode_key), pick(write, "rmw_kernel")
    probe_bytes = f_probe[1] * 16                      # grid size x 16-byte chunk
    k_fetch = probe_bytes / (f_probe[0] * 1024)        # true bytes per counted byte
    k_write = probe_bytes / (w_probe[0] * 1024)
    read_b = f_dec[0] * 1024 * k_fetch
    write_b = w_dec[0] * 1024 * k_write
    rec = {
        "kernel": decode_key + ", ...>",
        "kernel_source_sha256_16": kernel_source_hash(),
        "traffic_bytes_per_launch": read_b + write_b,
        "read_bytes_per_launch": read_b,
        "write_bytes_per_launch": write_b,
        "fetch_size_kib_per_launch": f_dec[0],
        "write_size_kib_per_launch": w_dec[0],
        "decode_dispatches": [f_dec[2], w_dec[2]],
        "calibration": {"probe": "kda_probe_rmw", "probe_bytes_each_way": probe_bytes,
                        "fetch_size_kib": f_probe[0], "write_size_kib": w_probe[0],
                        "fetch_scale": k_fetch, "write_scale": k_write},
    }
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
    return rec


def stored_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    if the kernel source changed since they were taken."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the chunked-prefill lines and print them as one JSON line "
                         "(for profiling the prefill kernel alone)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of this benchmark (FETCH_SIZE, then "
                         "WRITE_SIZE) into HBM bytes per decode launch, calibrated on the "
                         "probe kernel's dispatches, and write " + os.path.relpath(TRAFFIC_FILE, ROOT))
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from_counters(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the KDA decode step shards by stream with no "
              f"communication, so --gpus {args.gpus} is not run here.", file=sys.stderr)
        sys.exit(2)

    import torch

    import kda_synth
    from hybrid_linear_attention_kda_amd import kda
    kda.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.only_prefill:
        lines = [measure_prefill(M, L, sdt, max(5, args.steps // 20), 2) for M, L, sdt in PREFILL_SHAPES]
        print(json.dumps({"prefill": lines}), flush=True)
        return

    wl = kda_synth.WORKLOADS["glm_m32"]
    log(f"headline: {wl.description}; timed: {args.steps} steps after {args.warmup} warm-up steps, "
        f"a fresh input set for every timed step")
    # fresh q/k/v, alpha and beta for every timed step (input set k for timed step k)
    head = measure(wl, "f32", args.steps, args.warmup, n_inputs=args.steps, check=True)
    log(f"  {json.dumps({k: head[k] for k in ('launch', 'ms_per_step', 'ms_per_layer', 'state_GBps')})}")
    log(f"  timed pass parity: {json.dumps(head['timed_pass_parity'])}")

    secondary = []
    if not args.no_secondary:
        for name, sdt, mode in (("glm_m8", "f32", "plain"), ("glm_m8", "bf16", "plain"),
                                ("glm_m32", "bf16", "plain"),
                                ("glm_m128", "bf16", "plain"), ("glm_m1", "f32", "plain"),
                                ("glm_m32", "f32", "gated"), ("glm_m32", "f32", "layer"),
                                ("glm_m32", "f32", "multi"), ("glm_m128", "bf16", "multi")):
            w2 = kda_synth.WORKLOADS[name]
            if name == "glm_m1":
                w2 = kda_synth.Workload(**{**w2.__dict__, "layers": 34, "name": "glm_m1_34"})
            T = MULTI_T if mode == "multi" else 1
            r = measure(w2, sdt, max(20, args.steps // 4), args.warmup,
                        n_inputs=1 if mode == "multi" else min(w2.steps, 8), mode=mode, T=T)
            entry = {"workload": name if mode == "plain" else f"{name}_{mode}", "M": w2.M,
                     "input_sets": 1 if mode == "multi" else min(w2.steps, 8),
                     "layers": w2.layers, "state_dtype": sdt, "tokens_per_call": T,
                     "entry_point": {"plain": "kda_decode_step", "gated": "kda_decode_step_gated",
                                     "layer": "kda_decode_layer_step",
                                     "multi": "kda_decode_multi"}[mode],
                     "launch": r["launch"], "ms_per_layer": r["ms_per_layer"],
                     "ms_per_34_layer_step": r["ms_per_step"], "state_GBps": r["state_GBps"],
                     "frac_hbm_peak_state": r["state_GBps"] / HBM_PEAK_GBS,
                     "modes": r["modes"]}
            if mode == "multi":
                entry["us_per_token_layer"] = r["ms_per_layer"] * 1e3 / T
                entry["alg_GBps"] = r["modes"][r["launch"]]["alg_GBps"]
            secondary.append(entry)
            log(f"  {entry['workload']} {sdt} T={T}: {r['launch']} {r['ms_per_layer'] * 1e3:.2f} us/call "
                f"{r['state_GBps']:.0f} GB/s, algorithmic {r['modes'][r['launch']]['alg_GBps']:.0f} GB/s")
        for M, L, sdt in PREFILL_SHAPES:
            r = measure_prefill(M, L, sdt, max(5, args.steps // 20), 2)
            secondary.append(r)
            log(f"  {r['workload']} {sdt} ({r['form']}): {r['ms_per_layer']:.3f} ms/layer, "
                f"{r['us_per_token_layer'] * 1e3:.1f} ns/token-layer, {r['roofline']['achieved']:.1f} FP32-equivalent "
                f"TFLOP/s ({100 * r['roofline']['frac']:.1f}% of FP32 peak), bf16 MFMA "
                f"{100 * r['roofline']['bf16_mfma_frac']:.1f}% of peak, {r['roofline']['alg_GBps']:.0f} GB/s")

    ceiling = None
    if not args.no_ceiling:
        ceiling = stream_ceiling(wl.state_bytes("f32"), wl.layers, max(5, args.steps // 10))
        log(f"  probe ceiling: in-place rmw {ceiling['rmw']:.0f} GB/s, copy {ceiling['copy']:.0f} GB/s")

    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)

    avg_launch_s = head["ms_per_layer"] / 1e3
    achieved = head["alg_bytes_per_launch"] / avg_launch_s / 1e9
    roof = {
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        "traffic": stored_traffic(),
        "kernel": "decode_kernel<float, D=128, NSPLIT=1, NWAVES=16, VEC=4>",
        "alg_bytes_per_launch": head["alg_bytes_per_launch"],
        "avg_launch_us": avg_launch_s * 1e6,
    }
    out = {
        "metric": METRIC,
        "value": head["state_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "glm_m32: GLM-5.3-Flash KDA decode, M=32 streams, 34 layers with "
                               "distinct states, 64 heads x 128 x 128, FP32 state (4.25 GiB), "
                               "fresh q/k/v, alpha, beta every timed step",
                   "M": wl.M, "H": wl.H, "D": wl.D, "layers": wl.layers, "state_dtype": "f32",
                   "launch": head["launch"]},
        "ms_per_layer": head["ms_per_layer"],
        "frac_hbm_peak_state": head["state_GBps"] / HBM_PEAK_GBS,
        "modes": head["modes"],
        "timed_pass_parity": head["timed_pass_parity"],
        "stream_ceiling": None if ceiling is None else {
            "rmw_GBps": ceiling["rmw"], "copy_GBps": ceiling["copy"],
            "kernel": "kda_probe_rmw / kda_probe_copy: 512 threads, one 16-byte chunk per lane "
                      "(non-temporal load, non-temporal agent-scope store), one launch per "
                      "128 MiB layer chunk, 34 chunks",
            "decode_alg_over_rmw": achieved / ceiling["rmw"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
