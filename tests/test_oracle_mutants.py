"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of ``oracle/kda_oracle.c`` with one plausible mistake
(a dropped term, a wrong sign, a wrong index, a transposed operand, a wrong
tap order ...).  It is compiled into a temporary library and every pin of
``oracle_pins.ALL_PINS`` is run on it; at least one must fail.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "no_decay": [("S[(size_t)i * dv + j] *= alpha[i];", "S[(size_t)i * dv + j] *= 1.0;")],
    "decay_on_columns": [("S[(size_t)i * dv + j] *= alpha[i];", "S[(size_t)i * dv + j] *= alpha[j];")],
    "delta_sign": [("d[j] = beta * (v[j] - vhat);", "d[j] = beta * (v[j] + vhat);")],
    "no_beta": [("d[j] = beta * (v[j] - vhat);", "d[j] = (v[j] - vhat);")],
    "predict_transposed": [("vhat += S[(size_t)i * dv + j] * k[i];",
                            "vhat += S[(size_t)j * dv + i] * k[i];")],
    "read_with_k": [("acc += S[(size_t)i * dv + j] * q[i];", "acc += S[(size_t)i * dv + j] * k[i];")],
    "rank1_uses_q": [("S[(size_t)i * dv + j] += k[i] * d[j];", "S[(size_t)i * dv + j] += q[i] * d[j];")],
    "conv_taps_reversed": [("w[4 * (size_t)c + 0] * t0", "w[4 * (size_t)c + 3] * t0"),
                           ("w[4 * (size_t)c + 3] * xc", "w[4 * (size_t)c + 0] * xc")],
    "no_silu": [("z[c] = y / (1.0 + exp(-y));", "z[c] = y;")],
    "sigmoid_not_silu": [("z[c] = y / (1.0 + exp(-y));", "z[c] = 1.0 / (1.0 + exp(-y));")],
    "conv_state_not_shifted": [("cs_out[0 * (size_t)C + c] = t1;", "cs_out[0 * (size_t)C + c] = t0;")],
    "norm_no_sqrt": [("double r = 1.0 / sqrt(ss + eps);", "double r = 1.0 / (ss + eps);")],
    "norm_no_eps": [("double r = 1.0 / sqrt(ss + eps);", "double r = 1.0 / sqrt(ss);")],
    "norm_no_scale": [("out[i] = scale * x[i] * r;", "out[i] = x[i] * r;")],
    "q_from_k_channels": [("const double *zq = z + (size_t)mm * C + 0 * HD + (size_t)h * D;",
                           "const double *zq = z + (size_t)mm * C + 1 * HD + (size_t)h * D;")],
    "v_ignores_head": [("const double *zv = z + (size_t)mm * C + 2 * HD + (size_t)h * D;",
                        "const double *zv = z + (size_t)mm * C + 2 * HD;")],
    "k_scaled_like_q": [("kda_oracle_l2norm(D, zk, eps, 1.0, kh);\n        size_t u = (size_t)mm * H + h;\n"
                         "        kda_oracle_delta_step(D, D, S + u * (size_t)D * D, qh, kh, zv,\n"
                         "                              alpha + u * (size_t)D, beta[u], o + u * (size_t)D);\n"
                         "        free(qh);\n        free(kh);\n    }\n    free(z);",
                         "kda_oracle_l2norm(D, zk, eps, scale, kh);\n        size_t u = (size_t)mm * H + h;\n"
                         "        kda_oracle_delta_step(D, D, S + u * (size_t)D * D, qh, kh, zv,\n"
                         "                              alpha + u * (size_t)D, beta[u], o + u * (size_t)D);\n"
                         "        free(qh);\n        free(kh);\n    }\n    free(z);")],
    "gate_A_not_exponentiated": [("const double eA = exp(A_log);", "const double eA = A_log;")],
    "gate_bias_subtracted": [("const double xin = f[c] + dt_bias[c];", "const double xin = f[c] - dt_bias[c];")],
    "gate_bound_sign": [("g = kind == 0 ? lower_bound * sigmoid_d(eA * xin)",
                         "g = kind == 0 ? -lower_bound * sigmoid_d(eA * xin)")],
    "gate_log_space_alpha": [("alpha[c] = exp(g);", "alpha[c] = 1.0 + g;")],
    "gate_softplus_as_relu": [("return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));",
                               "return x > 0.0 ? x : 0.0;")],
    "gate_sigmoid_of_raw": [("g = kind == 0 ? lower_bound * sigmoid_d(eA * xin)",
                             "g = kind == 0 ? lower_bound * sigmoid_d(xin)")],
    "gate_A_of_first_head": [("kda_oracle_gate(D, f + u * (size_t)D, A_log[h],",
                              "kda_oracle_gate(D, f + u * (size_t)D, A_log[0],")],
    "gate_bias_ignores_head": [("A_log[h], dt_bias + h * (size_t)D, kind,", "A_log[h], dt_bias, kind,")],
    "beta_no_sigmoid": [("beta[i] = sigmoid_d(logit[i]);", "beta[i] = logit[i];")],
    "rmsnorm_sum_not_mean": [("const double r = 1.0 / sqrt(ss / D + eps);", "const double r = 1.0 / sqrt(ss + eps);")],
    "rmsnorm_no_gate": [("y[j] = o[j] * r * w[j] * sigmoid_d(g[j]);", "y[j] = o[j] * r * w[j];")],
    "rmsnorm_swish_gate": [("y[j] = o[j] * r * w[j] * sigmoid_d(g[j]);",
                            "y[j] = o[j] * r * w[j] * g[j] * sigmoid_d(g[j]);")],
    "rmsnorm_no_weight": [("y[j] = o[j] * r * w[j] * sigmoid_d(g[j]);", "y[j] = o[j] * r * sigmoid_d(g[j]);")],
    "layer_gate_of_other_head": [("og + u * (size_t)D, norm_w, norm_eps,", "og, norm_w, norm_eps,")],
    "multi_conv_state_not_carried": [("rc = kda_oracle_decode_step(1, H, D, Sm, xt, w, cm, cm, at, bt, scale, eps, ot);",
                                      "rc = kda_oracle_decode_step(1, H, D, Sm, xt, w, cs_in + (size_t)m * 3 * C, cm, at, bt, scale, eps, ot);")],
    "multi_alpha_of_first_token": [("memcpy(at, alpha + mt * HD, sizeof(double) * HD);",
                                    "memcpy(at, alpha + (size_t)m * T * HD, sizeof(double) * HD);")],
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    text = source
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, f"mutation site not unique for {name}: {old!r}"
        text = text.replace(old, new)
    src = tmp_path / f"mutant_{name}.c"
    src.write_text(text)
    lib = oracle.build(str(src), str(tmp_path / f"libmutant_{name}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
