"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutation edits the oracle's C source text (a sign, a dropped term, a
wrong operand, the readout order, the head mapping, the norm's mean or gate),
compiles the copy with gcc into a temporary directory and runs every pin on
it.  This shows the pins would notice such a slip in the oracle itself.  The
mistakes are planted only in this CPU copy; nothing here touches a GPU.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

UPDATE_BEGIN = "    /* S_t = a S_{t-1} - a b (S_{t-1} k_t) k_t^T + b v_t k_t^T */"
READOUT_BEGIN = "    /* o_t = scale * S_t q_t */"
READOUT_END = "        ot[i] = scale * acc;\n    }\n"


def _swap_readout_before_update(src: str) -> str:
    """Move the readout block in front of the state update (reads S_{t-1})."""
    u = src.index(UPDATE_BEGIN)
    r = src.index(READOUT_BEGIN)
    e = src.index(READOUT_END, r) + len(READOUT_END)
    update, readout = src[u:r], src[r:e]
    return src[:u] + readout + update + src[e:]


MUTATIONS = {
    "sign_of_delta_correction": [("upd -= a * b * sk[i]", "upd += a * b * sk[i]")],
    "dropped_write_term": [("upd += b * (double)vt[i] * kt[j];", "")],
    "dropped_beta_in_correction": [("upd -= a * b * sk[i]", "upd -= a * sk[i]")],
    "no_decay_on_state": [("double upd = a * s;", "double upd = s;")],
    "decay_sign": [("exp((double)g[", "exp(-(double)g[")],
    "readout_with_key": [("acc += S[(size_t)i * dk + j] * qt[j];",
                          "acc += S[(size_t)i * dk + j] * kt[j];")],
    "correction_uses_query": [("acc += S[(size_t)i * dk + j] * kt[j];\n        sk[i]",
                               "acc += S[(size_t)i * dk + j] * qt[j];\n        sk[i]")],
    "write_term_transposed_roles": [("upd += b * (double)vt[i] * kt[j];",
                                     "upd += b * (double)vt[j % dv] * kt[i % dk];")],
    "readout_unscaled": [("ot[i] = scale * acc;", "ot[i] = acc;")],
    "readout_before_update": "swap",
    "head_mapping_modulo": [("const int hk = h / (HV / H);", "const int hk = h % H;")],
    "norm_sum_not_mean": [("sqrt(ss / dv + eps)", "sqrt(ss + eps)")],
    "norm_gate_sigmoid": [("const double gate = zi / (1.0 + exp(-zi));",
                           "const double gate = 1.0 / (1.0 + exp(-zi));")],
    "norm_weight_dropped": [("* (double)w[i] * gate", "* gate")],
    "gate_sign": [("g[i] = -exp((double)A_log[h])", "g[i] = exp((double)A_log[h])")],
    "gate_scale_not_exponentiated": [("g[i] = -exp((double)A_log[h])",
                                      "g[i] = -(double)A_log[h]")],
    "gate_dt_bias_dropped": [("(dt_bias ? (double)dt_bias[h] : 0.0)", "0.0")],
    "softplus_as_relu": [(" + log1p(exp(-fabs(x)))", "")],
    "beta_of_negated_input": [("1.0 / (1.0 + exp(-(double)b_raw[i]))",
                               "1.0 / (1.0 + exp((double)b_raw[i]))")],
    "l2_eps_outside_sqrt": [("1.0 / sqrt(ss + eps)", "1.0 / (sqrt(ss) + eps)")],
    "l2_key_not_normalised": [("            l2norm_row(kd, dk, l2_eps);\n", "")],
    "slot_table_ignored": [("pool + ((size_t)s * HV + h) * ssz", "pool + ((size_t)n * HV + h) * ssz")],
    "skipped_sequence_output_unset": [("for (int i = 0; i < dv; ++i) ot[i] = 0.0;", "")],
    "layer_decay_sign": [("exp(g[p]), beta[p]", "exp(-g[p]), beta[p]")],
    "rope_interleaved_pairs": [("        y[i] = x[i] * c - x[i + half] * s;\n        y[i + half] = x[i + half] * c + x[i] * s;",
                                "        y[2 * i] = x[2 * i] * c - x[2 * i + 1] * s;\n        y[2 * i + 1] = x[2 * i + 1] * c + x[2 * i] * s;")],
    "rope_rotation_sign": [("y[i] = x[i] * c - x[i + half] * s;", "y[i] = x[i] * c + x[i + half] * s;"),
                           ("y[i + half] = x[i + half] * c + x[i] * s;", "y[i + half] = x[i + half] * c - x[i] * s;")],
    "rope_frequency": [("pow(theta, -2.0 * i / rd)", "pow(theta, -1.0 * i / rd)")],
    "attn_key_unrotated": [("rope_row(xd, d, rd, theta, (double)pos[n], kr);",
                            "for (int j = 0; j < d; ++j) kr[j] = xd[j];")],
    "attn_unscaled": [("sc[t] = scale * s;", "sc[t] = s;")],
    "attn_new_token_dropped": [("const int L = pos[n] + 1;", "const int L = pos[n] > 0 ? pos[n] : 1;")],
    "attn_gate_silu": [("v *= 1.0 / (1.0 + exp(-(double)gate[(size_t)p * d + j]));",
                        "v *= (double)gate[(size_t)p * d + j] / (1.0 + exp(-(double)gate[(size_t)p * d + j]));")],
    "attn_gqa_modulo": [("const int hk = h / (Hq / Hkv);", "const int hk = h % Hkv;")],
    "attn_new_value_from_cache": [("t < pos[n] ? vc + (kvh * Lmax + t) * d : vnew + kvh * d",
                                   "vc + (kvh * Lmax + t) * d")],
}


def _mutate(src: str, spec) -> str:
    if spec == "swap":
        return _swap_readout_before_update(src)
    for old, new in spec:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    return src


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    with open(oracle.SOURCE) as f:
        src = f.read()
    mutated = _mutate(src, MUTATIONS[name])
    assert mutated != src
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    lib = oracle.build(str(path), str(tmp_path / "libmutant.so"))
    orc = oracle.load(lib)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            failures.append((pin.__name__, str(e)[:80]))
    assert failures, f"mutation {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    """Control: the same build route without a mutation passes every pin."""
    lib = oracle.build(oracle.SOURCE, str(tmp_path / "libcopy.so"))
    orc = oracle.load(lib)
    for pin in oracle_pins.ALL_PINS:
        pin(orc)
