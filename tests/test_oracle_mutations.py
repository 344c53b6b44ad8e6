"""Plant plausible mistakes in copies of the oracle source and check that the pins catch each.

Each mutation is a textual edit of ``oracle/oracle.c`` compiled into a
temporary library (CPU only). A mutation that no pin detects would mean a
part of the oracle is not pinned.
"""
import os

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "kath_no_eps": ("den += eps;", "den += 0.0;"),
    "kath_elu_without_plus_one": ("x + 1.0 : exp(x)", "x + 1.0 : exp(x) - 1.0"),
    "kath_z_not_updated": ("z[i] += fk[i];", "z[i] += 0.0;"),
    "kath_phi_on_v_side": ("S[(size_t)i * dv + j] += fk[i] * v[j];",
                           "S[(size_t)i * dv + j] += k[i] * v[j];"),
    "gla_gate_after_write": ("g[i] * S[(size_t)i * dv + j] + k[i] * v[j]",
                             "g[i] * (S[(size_t)i * dv + j] + k[i] * v[j])"),
    "gla_gate_previous_token": ("gt = g + tok * dk;", "gt = g + (t > 0 ? tok - 1 : tok) * dk;"),
    "gdn_sign": ("u[j] = beta * (v[j] - alpha * pred);", "u[j] = beta * (v[j] + alpha * pred);"),
    "gdn_prediction_not_decayed": ("u[j] = beta * (v[j] - alpha * pred);",
                                   "u[j] = beta * (v[j] - pred);"),
    "gdn_no_beta": ("u[j] = beta * (v[j] - alpha * pred);", "u[j] = (v[j] - alpha * pred);"),
    "gdn_transposed_read": ("pred += S[(size_t)i * dv + j] * k[i];",
                            "pred += S[(size_t)j * dv + i] * k[i];"),
    "initial_state_ignored": ("if (S0) memcpy", "if (0) memcpy"),
    "kda_no_decay": ("for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= g[i];   /* decay first */",
                     "for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= 1.0;"),
    "kda_prediction_before_decay": (
        "        for (i = 0; i < dk; ++i)\n"
        "            for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= g[i];   /* decay first */\n"
        "        for (j = 0; j < dv; ++j) {\n"
        "            double pred = 0.0; /* (Sbar^T k_t)_j: what the decayed state recalls for k_t */\n"
        "            for (i = 0; i < dk; ++i) pred += S[(size_t)i * dv + j] * k[i];\n"
        "            u[j] = beta * (v[j] - pred);\n"
        "        }\n",
        "        for (j = 0; j < dv; ++j) {\n"
        "            double pred = 0.0;\n"
        "            for (i = 0; i < dk; ++i) pred += S[(size_t)i * dv + j] * k[i];\n"
        "            u[j] = beta * (v[j] - pred);\n"
        "        }\n"
        "        for (i = 0; i < dk; ++i)\n"
        "            for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= g[i];\n"),
    "kda_decay_transposed": ("S[(size_t)i * dv + j] *= g[i];", "S[(size_t)i * dv + j] *= g[j % dk];"),
    "kda_no_beta": ("u[j] = beta * (v[j] - pred);", "u[j] = (v[j] - pred);"),
    "ssd_decay_after_write": ("S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + k[i] * v[j];",
                              "S[(size_t)i * dv + j] = a * (S[(size_t)i * dv + j] + k[i] * v[j]);"),
    "ssd_gate_next_token": ("if (variant == OR_SSD) gt = g + tok;",
                            "if (variant == OR_SSD) gt = g + (t + 1 < N ? tok + 1 : tok);"),
    "ss_bbar_without_step": ("const double bbar = delta * Bm[tok * n + i];",
                             "const double bbar = Bm[tok * n + i];"),
    "ss_decay_sign": ("exp(delta * A[(size_t)d * n + i])", "exp(-delta * A[(size_t)d * n + i])"),
    "ss_state_index_reversed": ("exp(delta * A[(size_t)d * n + i])",
                                "exp(delta * A[(size_t)d * n + (n - 1 - i)])"),
    "ss_read_before_write": (
        "                h[i] = abar * h[i] + bbar * xt;\n            }\n"
        "            for (i = 0; i < n; ++i) acc += Cm[tok * n + i] * h[i];\n",
        "                acc += Cm[tok * n + i] * h[i];\n                h[i] = abar * h[i] + bbar * xt;\n"
        "            }\n"),
    "ss_output_reads_B": ("acc += Cm[tok * n + i] * h[i];", "acc += Bm[tok * n + i] * h[i];"),
    "ss_no_skip": ("y[tok * D + d] = acc + (Dskip ? Dskip[d] * xt : 0.0);", "y[tok * D + d] = acc;"),
    "ss_bias_dropped": ("double delta = dt[tok * D + d] + (dt_bias ? dt_bias[d] : 0.0);",
                        "double delta = dt[tok * D + d];"),
    "ss_softplus_ignored": ("if (dt_softplus) delta = softplus(delta);", "(void)dt_softplus;"),
    "ss_initial_state_ignored": ("if (h0) memcpy(h, h0", "if (0) memcpy(h, h0"),
    "bwd_decay_not_carried": ("for (j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= gi;",
                              "for (j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= 1.0;"),
    "bwd_output_path_missing": ("for (j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += q[i] * dO[j];",
                                "for (j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += 0.0 * dO[j];"),
    "bwd_delta_dp_sign": ("dp[j] = -beta * acc;", "dp[j] = beta * acc;"),
    "bwd_dbeta_without_prediction": ("db += acc * (v[j] - p[j]);", "db += acc * v[j];"),
    "bwd_dk_without_state_term": ("dk_[i] = acc + accp;", "dk_[i] = acc;"),
    "bwd_dalpha_on_decayed_state": ("acc += dsd * S_prev[(size_t)i * dv + j];",
                                    "acc += dsd * ai * S_prev[(size_t)i * dv + j];"),
    "bwd_kath_denominator_sign": ("dd -= dO[j] * o[j] / den;", "dd += dO[j] * o[j] / den;"),
    "bwd_kath_no_phi_derivative": ("dq[i] = dfq * (q[i] > 0.0 ? 1.0 : exp(q[i]));", "dq[i] = dfq;"),
    "bwd_gate_grad_post_state": (
        "for (j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * S_prev[(size_t)i * dv + j];",
        "for (j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * S_post[(size_t)i * dv + j];"),
    "kda_gate_previous_token": ("if (variant == OR_KDA) { gt = g + tok * dk;",
                                "if (variant == OR_KDA) { gt = g + (t > 0 ? tok - 1 : tok) * dk;"),
    "read_uses_key": ("for (i = 0; i < dk; ++i) acc += q[i] * S[(size_t)i * dv + j];\n            o[j] = acc;\n        }\n        c->state_read_macs += (uint64_t)dk * (uint64_t)dv;\n    } else {",
                      "for (i = 0; i < dk; ++i) acc += k[i] * S[(size_t)i * dv + j];\n            o[j] = acc;\n        }\n        c->state_read_macs += (uint64_t)dk * (uint64_t)dv;\n    } else {"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {name}"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = oracle.compile_library(str(mutated), str(tmp_path / f"liboracle_{name}.so"))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin detects the planted mistake {name}"
