"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of oracle/gdn_oracle.cpp with one plausible mistake (a
dropped term, a wrong sign, index or layout, a transposed operand, the other
reading of the decay order), compiled on the CPU into a temporary library. The
pins are then run against it. A mutant that passes every pin would show a blind
spot in the pins.
"""

import functools
import os
import subprocess

import pytest

import oracle
from oracle import gdn_oracle

from pins import ALL_PINS, golden_bf16_rounding, pin_bf16, pin_rollback

SK = "sk = sk + row[j] * static_cast<real>(k[at_qk(s, t, kh, j)]);"
DECAY = "row[j] = alpha * row[j];"
UPDATE = "row[j] = row[j] + d * static_cast<real>(k[at_qk(s, t, kh, j)]);"
Y = "y = y + row[j] * static_cast<real>(q[at_qk(s, t, kh, j)]);"

MUTANTS = {
    # The other reading of the decay order: sk from the undecayed state.
    "sk_before_decay": [(f"{DECAY}\n          {SK}", f"{SK}\n          {DECAY}")],
    "no_decay": [(DECAY, "row[j] = row[j];")],
    "exp_of_plus_g": [("return expf(-g);", "return expf(g);"),
                      ("exp(-static_cast<double>(g))", "exp(static_cast<double>(g))")],
    "delta_sign": [("(static_cast<real>(v[at_v(s, t, vh, i)]) - sk) * b",
                    "(sk - static_cast<real>(v[at_v(s, t, vh, i)])) * b")],
    "no_beta": [("- sk) * b;", "- sk);")],
    "beta_read_from_g": [("static_cast<real>(beta[at_scalar(s, t, vh)])",
                          "static_cast<real>(g[at_scalar(s, t, vh)])")],
    "y_before_update": [(f"{UPDATE}\n          {Y}", f"{Y}\n          {UPDATE}")],
    "y_reads_k": [(Y, Y.replace("(q[", "(k["))],
    "update_uses_q": [(UPDATE, UPDATE.replace("(k[", "(q["))],
    "sk_drops_last_term": [(SK, f"if (j + 1 < Dk) {SK}")],
    "y_drops_first_term": [(Y, f"if (j > 0) {Y}")],
    "head_maps_swapped": [("head_map == ORACLE_HEAD_MAP_MOD ? vh % Hk : vh / group_ratio",
                           "head_map == ORACLE_HEAD_MAP_MOD ? vh / group_ratio : vh % Hk")],
    "q_scale_ignored": [("output[at_v(s, t, vh, i)] = y * q_scale;",
                         "output[at_v(s, t, vh, i)] = y;")],
    "zero_bits_read_literally": [("if (bits == 0u) return 1.0f;",
                                  "if (bits == 0u) return 0.0f;")],
    "capture_tokens_reversed": [("capture[at_capture(s, t, vh, i, j)]",
                                 "capture[at_capture(s, T - 1 - t, vh, i, j)]")],
    "state_transposed": [("return ((s * Hv + vh) * Dv + i) * Dk + j;",
                          "return ((s * Hv + vh) * Dk + j) * Dv + i;")],
    "qk_token_head_swapped": [("return ((s * T + t) * Hk + kh) * Dk + j;",
                               "return ((s * Hk + kh) * T + t) * Dk + j;")],
    "v_token_head_swapped": [("return ((s * T + t) * Hv + vh) * Dv + i;",
                              "return ((s * Hv + vh) * T + t) * Dv + i;")],
    "scalar_token_head_swapped": [("return (s * T + t) * Hv + vh;",
                                   "return (s * Hv + vh) * T + t;")],
    "rollback_off_by_one": [("(s * p->n_tokens + accepted[s]) * head_state",
                             "(s * p->n_tokens + accepted[s] + 1) * head_state")],
    "rollback_ignores_bound": [("if (accepted[s] >= p->n_tokens) continue;",
                                "if (accepted[s] > p->n_tokens) continue;")],
    "bf16_truncates": [("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1;",
                        "")],
    "bf16_ties_away": [("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)")],
    "bf16_nan_not_quieted": [("return (uint16_t)((bits >> 16) | 0x0040u);",
                              "return (uint16_t)(bits >> 16);")],
    "bf16_v_not_widened": [("for (uint64_t e = 0; e < nv; ++e) vf[e] = bf16_to_f32(v[e]);",
                            "for (uint64_t e = 0; e < nv; ++e) vf[e] = (float)v[e];")],
    "state_in_ignored": [("X[i * Dk + j] = static_cast<real>(state_in[at_state(s, vh, i, j)]);",
                          "X[i * Dk + j] = 0;")],
    # Key normalisation option.
    "normk_no_eps": [("std::sqrt(ss + static_cast<real>(kNormEps))", "std::sqrt(ss)")],
    "normk_no_sqrt": [("real(1) / std::sqrt(ss + static_cast<real>(kNormEps))",
                       "real(1) / (ss + static_cast<real>(kNormEps))")],
    "normk_sum_abs": [("ss = ss + static_cast<real>(kr[j]) * static_cast<real>(kr[j]);",
                       "ss = ss + std::fabs(static_cast<real>(kr[j]));")],
    "normk_ignored": [("  if (!(options & kOptNormalizeK))\n", "  if (true)\n")],
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def build_mutant(name, edits, where):
    with open(gdn_oracle.SOURCE) as f:
        src = f.read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation {name}: pattern not unique: {old!r}"
        src = src.replace(old, new)
    cpp = os.path.join(where, f"{name}.cpp")
    lib = os.path.join(where, f"lib{name}.so")
    with open(cpp, "w") as f:
        f.write(src)
    subprocess.run(["g++", *gdn_oracle.CXXFLAGS, f"-I{gdn_oracle.HERE}", cpp, "-o", lib],
                   check=True)
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    lib = build_mutant(name, MUTANTS[name], str(mutant_dir))
    ref = functools.partial(oracle.reference, library=lib)
    extra = {pin_rollback: dict(rollback=functools.partial(oracle.rollback, library=lib)),
             pin_bf16: dict(ref_bf16=functools.partial(oracle.reference_bf16, library=lib)),
             golden_bf16_rounding: dict(to_bf16=functools.partial(oracle.to_bf16,
                                                                  library=lib))}
    caught = []
    for pin in ALL_PINS:
        try:
            pin(ref, **extra.get(pin, {}))
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passes every pin"
