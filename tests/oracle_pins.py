"""Pins that tie the CPU oracle to the pages and to mathematics, not to itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises ``AssertionError`` when
the oracle disagrees with something it must reproduce:

* values the pages print (the delta-rule worked example);
* an independent algorithm for the same quantity (the unrolled product form
  and the chunkwise WY/UT form of the recurrence);
* library routines for the special cases that reduce to them
  (torch's depthwise conv1d, SiLU and normalize, in float64);
* closed forms and invariants the pages state (exact recall, identity at
  alpha = 1 and beta = 0, the Householder contraction);
* the forget-gate table the pages print (keep factor, half-life, sigmoid
  output), torch's sigmoid and rms_norm for the write strength and the
  gated output norm.

``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py``
plants mistakes in a copy of the oracle's C source and checks that every
planted mistake makes at least one pin fail.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    den = max(float(np.max(np.abs(b))), 1e-300)
    err = float(np.max(np.abs(a - b))) / den if a.size else 0.0
    assert err <= rtol, f"{what}: relative error {err:.3e} > {rtol:.1e}"


def _unit(rng, n):
    k = rng.standard_normal(n)
    return k / np.linalg.norm(k)


# --------------------------------------------------------------------------
# 1. The pages' worked example ("GLM-5.3 deep dive", 8.2.2 step table)
# --------------------------------------------------------------------------
def _read_worked_example():
    rows = []
    with open(os.path.join(GOLDEN, "delta_rule_worked_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                tag, *vals = line.split()
                rows.append((tag, [float(v) for v in vals]))
    return rows


def pin_worked_example(orc):
    rows = _read_worked_example()
    writes = [v for t, v in rows if t == "write"]
    assert len(writes) == 3
    one = np.ones(2)
    S = np.zeros((2, 1))
    states = {}
    for step, k0, k1, val, s0, s1 in writes:
        k = np.array([k0, k1])
        S, _ = orc.delta_step(S, q=k, k=k, v=[val], alpha=one, beta=1.0)
        _close(S[:, 0], [s0, s1], 1e-12, f"worked example S after step {int(step)}")
        states[int(step)] = S.copy()
    for t, vals in rows:
        if t == "query_after":
            step, q0, q1, expect = vals
            Sq = states[int(step)]
            # a read is o = S^T q; beta = 0 and alpha = 1 leave S as it is
            _, o = orc.delta_step(Sq, q=[q0, q1], k=[1.0, 0.0], v=[0.0], alpha=one, beta=0.0)
            _close(o, [expect], 1e-12, f"worked example query after step {int(step)}")
        if t == "half_beta_step":
            step, beta, expect = vals
            k0, k1, val = writes[int(step) - 1][1:4]
            S_prev = states[int(step) - 1]
            S_half, _ = orc.delta_step(S_prev, q=[k0, k1], k=[k0, k1], v=[val],
                                       alpha=one, beta=beta)
            _close(S_half[0, 0], expect, 1e-12, "worked example with beta = 0.5")


# --------------------------------------------------------------------------
# 2. Brute force: the unrolled product form with explicit matrices
#    S_T = A_T..A_1 S_0 + sum_t A_T..A_{t+1} beta_t k_t v_t^T,
#    A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)      ("GLM-5.3 deep dive" Eq. 1)
# --------------------------------------------------------------------------
def _unrolled(S0, ks, vs, alphas, betas, T):
    dk = S0.shape[0]
    A = [(np.eye(dk) - b * np.outer(k, k)) @ np.diag(a) for k, a, b in zip(ks, alphas, betas)]
    P = np.eye(dk)
    for t in range(T):
        P = A[t] @ P
    S = P @ S0
    for t in range(T):
        P = np.eye(dk)
        for r in range(t + 1, T):
            P = A[r] @ P
        S = S + P @ (betas[t] * np.outer(ks[t], vs[t]))
    return S


def pin_unrolled_product(orc, dk=5, dv=3, T=6, seed=11):
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((dk, dv))
    ks = [_unit(rng, dk) for _ in range(T)]
    qs = [rng.standard_normal(dk) for _ in range(T)]
    vs = [rng.standard_normal(dv) for _ in range(T)]
    alphas = [rng.uniform(0.2, 1.0, dk) for _ in range(T)]
    betas = [float(rng.uniform(0.0, 1.0)) for _ in range(T)]
    S = S0.copy()
    for t in range(T):
        S, o = orc.delta_step(S, qs[t], ks[t], vs[t], alphas[t], betas[t])
        ref = _unrolled(S0, ks, vs, alphas, betas, t + 1)
        _close(S, ref, 1e-12, f"unrolled form, state after step {t + 1}")
        _close(o, ref.T @ qs[t], 1e-12, f"unrolled form, output at step {t + 1}")


# --------------------------------------------------------------------------
# 3. Independent algorithm: the chunkwise WY representation + UT transform
#    ("GLM-5.3 deep dive" 8.2.5, Eq. 6-9).  Gamma_r is the inclusive
#    cumulative decay; gamma^{i->C} excludes token i; StrictTril inside the
#    inverse; Tril (with the diagonal) for the output.
# --------------------------------------------------------------------------
def _chunk_wy(S, K, Q, V, Alpha, beta):
    C = K.shape[0]
    G = np.cumprod(Alpha, axis=0)                   # Gamma [C, dk]
    GK, KG, GQ = G * K, K / G, G * Q
    Mx = np.linalg.inv(np.eye(C) + np.tril(np.diag(beta) @ GK @ KG.T, -1)) @ np.diag(beta)
    W, U = Mx @ GK, Mx @ V
    Delta = U - W @ S
    O = GQ @ S + np.tril(GQ @ KG.T) @ Delta
    S_next = np.diag(G[-1]) @ S + ((G[-1] / G) * K).T @ Delta
    return S_next, O


def pin_chunk_form(orc, dk=16, dv=16, C=16, seed=12):
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((dk, dv)) * 0.1
    K = np.stack([_unit(rng, dk) for _ in range(C)])
    Q = rng.standard_normal((C, dk))
    V = rng.standard_normal((C, dv))
    Alpha = rng.uniform(0.5, 1.0, (C, dk))
    beta = rng.uniform(0.0, 1.0, C)
    S_ref, O_ref = _chunk_wy(S0, K, Q, V, Alpha, beta)
    S = S0.copy()
    O = np.empty((C, dv))
    for t in range(C):
        S, O[t] = orc.delta_step(S, Q[t], K[t], V[t], Alpha[t], beta[t])
    _close(S, S_ref, 1e-11, "chunk WY form, final state")
    _close(O, O_ref, 1e-11, "chunk WY form, outputs")


# --------------------------------------------------------------------------
# 4. Invariants stated by the pages
# --------------------------------------------------------------------------
def pin_identity_alpha1_beta0(orc, seed=13):
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((8, 6))
    q = rng.standard_normal(8)
    S, o = orc.delta_step(S0, q, _unit(rng, 8), rng.standard_normal(6), np.ones(8), 0.0)
    assert np.array_equal(S, S0), "alpha = 1, beta = 0 must leave S unchanged bit for bit"
    _close(o, S0.T @ q, 1e-14, "alpha = 1, beta = 0 readout")


def pin_pure_decay_beta0(orc, seed=14):
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((8, 6))
    a = rng.uniform(0, 1, 8)
    S, _ = orc.delta_step(S0, np.zeros(8), _unit(rng, 8), rng.standard_normal(6), a, 0.0)
    assert np.array_equal(S, S0 * a[:, None]), "beta = 0 must be a pure row decay"


def pin_exact_recall(orc, seed=15):
    """beta = 1 and a unit key: querying with that key returns v, whatever the
    fade did ("GLM-5.3 deep dive" 8.2.3)."""
    rng = np.random.default_rng(seed)
    for dk, dv in ((2, 1), (7, 5), (16, 16)):
        S0 = rng.standard_normal((dk, dv))
        k = _unit(rng, dk)
        v = rng.standard_normal(dv)
        S, o = orc.delta_step(S0, k, k, v, rng.uniform(0, 1, dk), 1.0)
        _close(o, v, 1e-13, f"exact recall dk={dk}")
        _close(S.T @ k, v, 1e-13, f"exact recall via S^T k, dk={dk}")


def pin_exact_recall_rational(orc):
    """A Pythagorean unit key (3, 4, 12)/13 with rational alpha and state: the
    recall with beta = 1 is exactly v, and the corrected state is known
    exactly in rationals; the double oracle must agree to rounding."""
    k = [Fraction(3, 13), Fraction(4, 13), Fraction(12, 13)]
    S0 = [[Fraction(1, 2), Fraction(-1, 4)], [Fraction(3, 8), Fraction(1)], [Fraction(-2), Fraction(1, 16)]]
    v = [Fraction(5, 4), Fraction(-3, 2)]
    alpha = [Fraction(1, 2), Fraction(3, 4), Fraction(7, 8)]
    # exact: faded state, prediction, corrected state, recall with beta = 1
    Sf = [[alpha[i] * S0[i][j] for j in range(2)] for i in range(3)]
    S_exact = [[Sf[i][j] + k[i] * (v[j] - sum(Sf[r][j] * k[r] for r in range(3)))
                for j in range(2)] for i in range(3)]
    S, o = orc.delta_step(np.array(S0, float), [float(x) for x in k], [float(x) for x in k],
                          [float(x) for x in v], [float(x) for x in alpha], 1.0)
    _close(o, [float(x) for x in v], 1e-14, "rational exact recall")
    _close(S, np.array(S_exact, float), 1e-14, "rational corrected state")


def pin_contraction(orc, seed=16):
    """With |k| = 1 and beta in [0,1], I - beta k k^T has eigenvalue 1 - beta
    along k and 1 elsewhere, so |S' - beta k v^T|_F <= |Diag(alpha) S|_F."""
    rng = np.random.default_rng(seed)
    for _ in range(20):
        dk, dv = 6, 4
        S0 = rng.standard_normal((dk, dv))
        k = _unit(rng, dk)
        v = rng.standard_normal(dv)
        a = rng.uniform(0, 1, dk)
        b = float(rng.uniform(0, 1))
        S, _ = orc.delta_step(S0, np.zeros(dk), k, v, a, b)
        lhs = np.linalg.norm(S - b * np.outer(k, v))
        rhs = np.linalg.norm(a[:, None] * S0)
        assert lhs <= rhs * (1 + 1e-12), f"contraction violated: {lhs} > {rhs}"


def pin_column_permutation(orc, seed=17):
    """Value columns are independent: permuting them permutes S and o."""
    rng = np.random.default_rng(seed)
    dk, dv = 6, 5
    S0 = rng.standard_normal((dk, dv))
    q, k, v = rng.standard_normal(dk), _unit(rng, dk), rng.standard_normal(dv)
    a = rng.uniform(0, 1, dk)
    perm = rng.permutation(dv)
    S1, o1 = orc.delta_step(S0, q, k, v, a, 0.7)
    S2, o2 = orc.delta_step(S0[:, perm], q, k, v[perm], a, 0.7)
    _close(S2, S1[:, perm], 1e-14, "column permutation, state")
    _close(o2, o1[perm], 1e-14, "column permutation, output")


# --------------------------------------------------------------------------
# 5. Convolution and SiLU against torch's depthwise conv1d and silu (float64)
#    ("GLM-5.3 deep dive" 8.2.4 step 2; "At the 262k cap ...", "Geometry")
# --------------------------------------------------------------------------
def pin_conv_library(orc, C=12, T=7, seed=18):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((C, 4))
    cs0 = rng.standard_normal((3, C))
    xs = rng.standard_normal((T, C))
    # torch: the three cached taps stand in for the causal left padding
    seq = torch.from_numpy(np.concatenate([cs0, xs], 0).T[None])           # [1, C, 3+T]
    y = F.conv1d(seq, torch.from_numpy(w)[:, None, :], groups=C)[0].T       # [T, C]
    z_ref = F.silu(y).numpy()
    cs = cs0
    for t in range(T):
        z, cs_next = orc.conv_silu(xs[t], w, cs)
        _close(z, z_ref[t], 1e-13, f"conv+SiLU vs torch conv1d, token {t}")
        assert np.array_equal(cs_next, np.concatenate([cs0, xs], 0)[t + 1:t + 4]), \
            "conv state must hold the last three raw inputs, oldest first"
        cs = cs_next


def pin_conv_closed_forms(orc, C=8, seed=19):
    rng = np.random.default_rng(seed)
    # one-hot on the current tap: y = x
    w = np.zeros((C, 4))
    w[:, 3] = 1.0
    x = rng.standard_normal(C)
    z, _ = orc.conv_silu(x, w, rng.standard_normal((3, C)))
    _close(z, F.silu(torch.from_numpy(x)).numpy(), 1e-15, "one-hot current tap")
    # impulse response: tap 3 - t is what a unit impulse t tokens ago sees
    w = rng.standard_normal((C, 4))
    cs = np.zeros((3, C))
    for t in range(4):
        xt = np.ones(C) if t == 0 else np.zeros(C)
        z, cs = orc.conv_silu(xt, w, cs)
        _close(z, F.silu(torch.from_numpy(w[:, 3 - t].copy())).numpy(), 1e-15,
               f"impulse response, {t} tokens after")
    # SiLU closed values: SiLU(0) = 0 and SiLU(y) - SiLU(-y) = y
    w = np.zeros((C, 4))
    w[:, 3] = 1.0
    y = np.linspace(-6, 6, C)
    zp, _ = orc.conv_silu(y, w, np.zeros((3, C)))
    zn, _ = orc.conv_silu(-y, w, np.zeros((3, C)))
    _close(zp - zn, y, 1e-15, "SiLU odd part")
    z0, _ = orc.conv_silu(np.zeros(C), w, np.zeros((3, C)))
    assert np.all(z0 == 0.0)


# --------------------------------------------------------------------------
# 6. L2 norm ("GLM-5.3 deep dive" 8.2.6, epsilon 1e-6)
# --------------------------------------------------------------------------
def pin_l2norm(orc, seed=20):
    _close(orc.l2norm([3.0, 4.0], eps=0.0), [0.6, 0.8], 1e-15, "l2norm (3,4)")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(128)
    ref = F.normalize(torch.from_numpy(x), dim=0, eps=0.0).numpy()
    _close(orc.l2norm(x, eps=0.0), ref, 1e-15, "l2norm vs torch normalize")
    _close(orc.l2norm(x, eps=0.0, scale=0.25), 0.25 * ref, 1e-15, "l2norm scale")
    # epsilon: (1e-4, 0) -> 1e-4 / sqrt(1e-8 + 1e-6)
    _close(orc.l2norm([1e-4, 0.0], eps=1e-6), [1e-4 / math.sqrt(1.01e-6), 0.0], 1e-15,
           "l2norm epsilon")
    assert np.all(orc.l2norm(np.zeros(5), eps=1e-6) == 0.0)


# --------------------------------------------------------------------------
# 7. End to end on tiny inputs: the fused step against a composition of
#    torch conv1d + silu + normalize (eps = 0 on both sides) and the unrolled
#    product form, over several tokens, streams and heads.
# --------------------------------------------------------------------------
def pin_decode_step_end_to_end(orc, M=2, H=3, D=4, T=5, seed=21):
    rng = np.random.default_rng(seed)
    HD, C = H * D, 3 * H * D
    S0 = rng.standard_normal((M, H, D, D)) * 0.1
    w = rng.standard_normal((C, 4)) * 0.5
    cs0 = rng.standard_normal((M, 3, C))
    xs = rng.standard_normal((T, M, 3, HD))
    alphas = rng.uniform(0.3, 1.0, (T, M, H, D))
    betas = rng.uniform(0.0, 1.0, (T, M, H))
    scale = 1.0 / math.sqrt(D)

    S, cs = S0.copy(), cs0.copy()
    outs = []
    for t in range(T):
        S, cs, o = orc.decode_step(S, xs[t], w, cs, alphas[t], betas[t], scale, eps=0.0)
        outs.append(o)

    for m in range(M):
        seq = np.concatenate([cs0[m], xs[:, m].reshape(T, C)], 0)            # [3+T, C]
        y = F.conv1d(torch.from_numpy(seq.T[None]), torch.from_numpy(w)[:, None, :], groups=C)
        z = F.silu(y)[0].T.numpy().reshape(T, 3, H, D)
        for h in range(H):
            q = F.normalize(torch.from_numpy(z[:, 0, h]), dim=1, eps=0.0).numpy() * scale
            k = F.normalize(torch.from_numpy(z[:, 1, h]), dim=1, eps=0.0).numpy()
            v = z[:, 2, h]
            for t in range(T):
                ref = _unrolled(S0[m, h], list(k), list(v), list(alphas[:, m, h]),
                                list(betas[:, m, h]), t + 1)
                _close(outs[t][m, h], ref.T @ q[t], 1e-12, f"end to end o, m={m} h={h} t={t}")
            _close(S[m, h], ref, 1e-12, f"end to end state, m={m} h={h}")
        assert np.array_equal(cs[m], seq[T:T + 3]), "end to end conv state"


def pin_recurrent_matches_decode(orc, M=2, H=2, D=8, seed=22):
    """The recurrent entry from post-conv q|k|v equals the fused step fed the
    conv output, with the conv taken from torch."""
    rng = np.random.default_rng(seed)
    HD, C = H * D, 3 * H * D
    S0 = rng.standard_normal((M, H, D, D))
    w = rng.standard_normal((C, 4))
    cs0 = rng.standard_normal((M, 3, C))
    x = rng.standard_normal((M, 3, HD))
    a = rng.uniform(0, 1, (M, H, D))
    b = rng.uniform(0, 1, (M, H))
    S1, _, o1 = orc.decode_step(S0, x, w, cs0, a, b, 0.5)
    seq = np.concatenate([cs0, x.reshape(M, 1, C)], 1)                       # [M, 4, C]
    y = F.conv1d(torch.from_numpy(seq.transpose(0, 2, 1).reshape(1, M * C, 4)),
                 torch.from_numpy(np.tile(w, (M, 1)))[:, None, :], groups=M * C)
    qkv = F.silu(y).numpy().reshape(M, 3, HD)
    S2, o2 = orc.recurrent_step(S0, qkv, a, b, 0.5)
    _close(S2, S1, 1e-14, "recurrent vs fused state")
    _close(o2, o1, 1e-14, "recurrent vs fused output")


def pin_unit_independence(orc, M=3, H=4, D=8, seed=23):
    """Streams and heads are independent: changing one (stream, head)'s inputs
    changes only that unit's state and output."""
    rng = np.random.default_rng(seed)
    HD, C = H * D, 3 * H * D
    S0 = rng.standard_normal((M, H, D, D))
    w = rng.standard_normal((C, 4))
    cs0 = rng.standard_normal((M, 3, C))
    x = rng.standard_normal((M, 3, HD))
    a = rng.uniform(0, 1, (M, H, D))
    b = rng.uniform(0, 1, (M, H))
    S1, _, o1 = orc.decode_step(S0, x, w, cs0, a, b, 0.3)
    m0, h0 = 1, 2
    x2 = x.copy()
    x2[m0, :, h0 * D:(h0 + 1) * D] += 1.0
    a2 = a.copy()
    a2[m0, h0] *= 0.5
    S2, _, o2 = orc.decode_step(S0, x2, w, cs0, a2, b, 0.3)
    for m in range(M):
        for h in range(H):
            same = (m, h) != (m0, h0)
            assert np.array_equal(S1[m, h], S2[m, h]) == same, f"state unit ({m},{h})"
            assert np.array_equal(o1[m, h], o2[m, h]) == same, f"output unit ({m},{h})"


# --------------------------------------------------------------------------
# 5. Forget gate, write strength, gated RMSNorm ("GLM-5.3 deep dive" 8.2.3,
#    8.2.4)
# --------------------------------------------------------------------------
def _read_gate_table():
    rows, neutral = [], None
    with open(os.path.join(GOLDEN, "gate_half_life.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tag, *vals = line.split()
            if tag == "row":
                rows.append((vals[0], vals[1], vals[2]))
            elif tag == "neutral":
                neutral = [float(v) for v in vals]
    return rows, neutral


def _logit(p):
    return math.log(p) - math.log1p(-p)


def pin_gate_table(orc):
    """Every row of the pages' table, at A_h = 0 (Miles' initial value): the
    sigmoid output s is produced by f + b = logit(s); the oracle's alpha must
    round to the printed keep factor and its half-life to the printed one."""
    rows, neutral = _read_gate_table()
    assert len(rows) == 5 and neutral is not None
    for alpha_txt, half_txt, s_txt in rows:
        x = 50.0 if s_txt == "to1" else _logit(float(s_txt))
        a = float(orc.gate(np.array([x]), 0.0, np.array([0.0]), kind=0, lower_bound=-5.0)[0])
        digits = len(alpha_txt.split(".")[1])
        assert round(a, digits) == float(alpha_txt), f"alpha {a} for s={s_txt}, printed {alpha_txt}"
        half = math.log(0.5) / math.log(a)
        if half_txt == "under1":
            assert 0 < half < 1, f"half-life {half} for printed alpha {alpha_txt}"
        else:
            assert int(half) == int(half_txt), f"half-life {half} for printed {half_txt}"
    A, fb, g, alpha = neutral
    a = float(orc.gate(np.array([fb]), A, np.array([0.0]), kind=0, lower_bound=-5.0)[0])
    assert abs(math.log(a) - g) < 1e-12 and round(a, 3) == alpha, f"neutral point {a}"
    # the floor: alpha stays above exp(-5) for any input, and reaches it in the limit
    big = orc.gate(np.array([-80.0, 0.0, 80.0]), 0.0, np.zeros(3))
    assert np.all(big >= math.exp(-5.0)) and np.all(big <= 1.0)
    assert abs(big[2] - math.exp(-5.0)) < 1e-15 and big[0] > 1.0 - 1e-15


def pin_gate_structure(orc, seed=30):
    """The gate reads f and dt_bias only through f + b: (f, b, A) and
    (f - c, b + c, A) agree.  exp(A_h) scales the sigmoid's input in the
    bounded form (A = ln 2 at x/2 equals A = 0 at x) and the log-decay in
    the softplus form (A = ln 2 squares alpha).  Alpha falls as f + b grows."""
    rng = np.random.default_rng(seed)
    f = rng.standard_normal(16) * 3
    b = rng.standard_normal(16)
    c = rng.standard_normal(16)
    for kind in (0, 1):
        a1 = orc.gate(f, 0.3, b, kind=kind)
        a2 = orc.gate(f - c, 0.3, b + c, kind=kind)
        _close(a1, a2, 1e-14, f"gate kind {kind}: shift between f and dt_bias")
        if kind == 0:      # exp(A) multiplies the sigmoid's input
            a3 = orc.gate((f + b) / 2, math.log(2.0), np.zeros(16), kind=kind)
            a4 = orc.gate(f + b, 0.0, np.zeros(16), kind=kind)
        else:              # exp(A) multiplies the log-decay: alpha is raised to exp(A)
            a3 = orc.gate(f + b, math.log(2.0), np.zeros(16), kind=kind)
            a4 = orc.gate(f + b, 0.0, np.zeros(16), kind=kind) ** 2
        _close(a3, a4, 1e-14, f"gate kind {kind}: how exp(A_log) enters")
        xs = np.linspace(-6, 6, 25)
        al = orc.gate(xs, 0.0, np.zeros(25), kind=kind)
        assert np.all(np.diff(al) < 0) and np.all((al > 0) & (al < 1)), f"gate kind {kind} monotone in (0, 1)"


def pin_gate_softplus_closed_form(orc, seed=31):
    """fla's default gate exp(-exp(A) softplus(x)) is sigmoid(-x) ** exp(A);
    at A = 0 it is the tiny workload's alpha = exp(-softplus(g)) = 1/(1+e^g)."""
    rng = np.random.default_rng(seed)
    xs = rng.standard_normal(20) * 4
    for A in (0.0, -0.7, 1.3):
        got = orc.gate(xs, A, np.zeros(20), kind=1)
        want = np.array([(1.0 / (1.0 + math.exp(x))) ** math.exp(A) for x in xs])
        _close(got, want, 1e-13, f"softplus gate at A={A}")
    # no overflow far out: softplus(800) = 800
    far = orc.gate(np.array([800.0, -800.0]), 0.0, np.zeros(2), kind=1)
    assert far[0] == 0.0 and far[1] == 1.0


def pin_beta_sigmoid(orc, seed=32):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(50) * 5
    got = orc.beta(z)
    _close(got, torch.sigmoid(torch.tensor(z, dtype=torch.float64)).numpy(), 1e-15, "beta vs torch.sigmoid")
    assert orc.beta(np.array([0.0]))[0] == 0.5
    _close(orc.beta(z) + orc.beta(-z), np.ones(50), 1e-15, "sigmoid(x) + sigmoid(-x) = 1")


def pin_gated_rmsnorm(orc, D=128, seed=33):
    """torch's rms_norm (float64) times torch.sigmoid of the gate; a constant
    vector normalises to c/sqrt(c^2 + eps); without eps the norm ignores the
    scale of o and flips with its sign."""
    rng = np.random.default_rng(seed)
    o = rng.standard_normal(D) * 0.3
    g = rng.standard_normal(D) * 2
    w = 1.0 + 0.1 * rng.standard_normal(D)
    ot, gt, wt = (torch.tensor(v, dtype=torch.float64) for v in (o, g, w))
    want = (F.rms_norm(ot, (D,), weight=wt, eps=1e-5) * torch.sigmoid(gt)).numpy()
    _close(orc.gated_rmsnorm(o, g, w, eps=1e-5), want, 1e-14, "gated rmsnorm vs torch")
    c = 0.01
    y = orc.gated_rmsnorm(np.full(D, c), np.zeros(D), np.ones(D), eps=1e-5)
    _close(y, np.full(D, 0.5 * c / math.sqrt(c * c + 1e-5)), 1e-14, "constant vector")
    y1 = orc.gated_rmsnorm(o, g, w, eps=0.0)
    _close(orc.gated_rmsnorm(7.5 * o, g, w, eps=0.0), y1, 1e-14, "scale invariance")
    _close(orc.gated_rmsnorm(-o, g, w, eps=0.0), -y1, 1e-14, "sign")


def _gate_inputs(rng, M, H, D):
    f = rng.standard_normal((M, H * D))
    A = rng.uniform(-0.5, 0.5, H)
    b = rng.normal(-4.0, 1.5, H * D)
    bl = rng.standard_normal((M, H))
    return f, A, b, bl


def pin_gated_step_wiring(orc, M=2, H=3, D=8, seed=34):
    """decode_step_gated = decode_step with alpha from each (stream, head)'s
    own f, A_log[h], dt_bias[h] and beta = sigmoid(logit); layer_step = its
    outputs through the gated RMSNorm of each head with out_gate of that
    (stream, head).  Heads get distinct gate parameters so a wrong index shows."""
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((M, H, D, D)) * 0.1
    x = rng.standard_normal((M, 3, H * D))
    w = rng.standard_normal((3 * H * D, 4)) * 0.5
    cs = rng.standard_normal((M, 3, 3 * H * D))
    f, A, b, bl = _gate_inputs(rng, M, H, D)
    og = rng.standard_normal((M, H * D))
    nw = 1.0 + 0.1 * rng.standard_normal(D)
    for kind, lb in ((0, -5.0), (1, 0.0)):
        alpha = np.empty((M, H, D))
        for m in range(M):
            for h in range(H):
                fb = f[m, h * D:(h + 1) * D] + b[h * D:(h + 1) * D]
                if kind == 0:
                    g = lb / (1.0 + np.exp(-np.exp(A[h]) * fb))
                else:
                    g = -np.exp(A[h]) * np.log1p(np.exp(fb))
                alpha[m, h] = np.exp(g)
        beta = 1.0 / (1.0 + np.exp(-bl))
        S1, cs1, o1 = orc.decode_step(S, x, w, cs, alpha, beta, 0.25)
        S2, cs2, o2 = orc.decode_step_gated(S, x, w, cs, f, A, b, bl, 0.25, kind=kind, lower_bound=lb)
        _close(S2, S1, 1e-13, f"gated step state, kind {kind}")
        _close(o2, o1, 1e-13, f"gated step output, kind {kind}")
        assert np.array_equal(cs1, cs2)
        S3, cs3, y = orc.layer_step(S, x, w, cs, f, A, b, bl, 0.25, og, nw, kind=kind, lower_bound=lb)
        _close(S3, S1, 1e-13, f"layer step state, kind {kind}")
        ot = torch.tensor(o1.reshape(M * H, D), dtype=torch.float64)
        gt = torch.tensor(og.reshape(M * H, D), dtype=torch.float64)
        want = F.rms_norm(ot, (D,), weight=torch.tensor(nw, dtype=torch.float64), eps=1e-5) * torch.sigmoid(gt)
        _close(y.reshape(M * H, D), want.numpy(), 1e-13, f"layer step output, kind {kind}")


# --------------------------------------------------------------------------
# 6. T tokens per call ("GLM-5.3 deep dive" 8.2.6: fla's decode mode loops
#    over the tokens of a short input)
# --------------------------------------------------------------------------
def pin_multi_token(orc, M=2, H=2, D=8, T=5, seed=40):
    """decode_multi over T tokens equals T single steps (state, conv state and
    every token's output), and its recurrence part equals the chunkwise
    WY/UT form of the deep dive's 8.2.5 over the same T tokens."""
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((M, H, D, D)) * 0.1
    x = rng.standard_normal((M, T, 3, H * D))
    w = rng.standard_normal((3 * H * D, 4)) * 0.5
    cs0 = rng.standard_normal((M, 3, 3 * H * D))
    alpha = rng.uniform(0.5, 1.0, (M, T, H, D))
    beta = rng.uniform(0.0, 1.0, (M, T, H))
    S1, cs1, o1 = orc.decode_multi(S0, x, w, cs0, alpha, beta, 0.3)
    S, cs = S0, cs0
    for t in range(T):
        S, cs, o = orc.decode_step(S, x[:, t], w, cs, alpha[:, t], beta[:, t], 0.3)
        _close(o1[:, t], o, 1e-14, f"token {t} output")
    _close(S1, S, 1e-14, "state after T tokens")
    assert np.array_equal(cs1, cs), "conv state after T tokens"
    # the recurrence alone: q, k, v of one (stream, head) through the chunk form
    m, h = 1, 1
    cs_t = cs0[m]
    Q, K, V = [], [], []
    for t in range(T):
        zz, cs_t = orc.conv_silu(x[m, t].reshape(-1), w, cs_t)
        zz = zz.reshape(3, H, D)[:, h]
        Q.append(orc.l2norm(zz[0], scale=0.3))
        K.append(orc.l2norm(zz[1]))
        V.append(zz[2])
    Sc, Oc = _chunk_wy(S0[m, h], np.array(K), np.array(Q), np.array(V), alpha[m, :, h], beta[m, :, h])
    _close(S1[m, h], Sc, 1e-12, "state vs chunk form")
    _close(o1[m, :, h], Oc, 1e-12, "outputs vs chunk form")


def pin_sequence_gated(orc, M=2, H=3, D=8, T=6, seed=41):
    """sequence_gated over T tokens = T single gated steps, and = the
    ungated multi-token call fed with the gate's alpha and sigmoid(logit)."""
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((M, H, D, D)) * 0.1
    x = rng.standard_normal((M, T, 3, H * D))
    w = rng.standard_normal((3 * H * D, 4)) * 0.5
    cs0 = rng.standard_normal((M, 3, 3 * H * D))
    f = rng.standard_normal((M, T, H * D))
    A = rng.uniform(-0.5, 0.5, H)
    b = rng.normal(-4.0, 1.0, H * D)
    bl = rng.standard_normal((M, T, H))
    S1, cs1, o1 = orc.sequence_gated(S0, x, w, cs0, f, A, b, bl, 0.3, lower_bound=-5.0)
    S, cs = S0, cs0
    for t in range(T):
        S, cs, o = orc.decode_step_gated(S, x[:, t], w, cs, f[:, t], A, b, bl[:, t], 0.3, lower_bound=-5.0)
        _close(o1[:, t], o, 1e-14, f"gated token {t}")
    _close(S1, S, 1e-14, "gated sequence state")
    assert np.array_equal(cs1, cs)
    alpha = np.empty((M, T, H, D))
    for m in range(M):
        for t in range(T):
            for h in range(H):
                alpha[m, t, h] = orc.gate(f[m, t, h * D:(h + 1) * D], A[h], b[h * D:(h + 1) * D])
    S2, _, o2 = orc.decode_multi(S0, x, w, cs0, alpha, orc.beta(bl), 0.3)
    _close(S2, S1, 1e-14, "gated sequence vs multi with gate alpha")
    _close(o2, o1, 1e-14, "gated sequence outputs vs multi")


ALL_PINS = [
    pin_worked_example,
    pin_unrolled_product,
    pin_chunk_form,
    pin_identity_alpha1_beta0,
    pin_pure_decay_beta0,
    pin_exact_recall,
    pin_exact_recall_rational,
    pin_contraction,
    pin_column_permutation,
    pin_conv_library,
    pin_conv_closed_forms,
    pin_l2norm,
    pin_decode_step_end_to_end,
    pin_recurrent_matches_decode,
    pin_unit_independence,
    pin_gate_table,
    pin_gate_structure,
    pin_gate_softplus_closed_form,
    pin_beta_sigmoid,
    pin_gated_rmsnorm,
    pin_gated_step_wiring,
    pin_multi_token,
    pin_sequence_gated,
]
