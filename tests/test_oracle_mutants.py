"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake (a dropped term, a wrong sign, a wrong index, a
swapped operand, an off-by-one comparison) in a private copy of the oracle's
C source, builds it on the CPU, and checks that at least one pin in
test_oracle_pins.py fails against it.  The committed oracle is untouched.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dlm_oracle.c")

MUTANTS = [
    ("kl_sign", "d += exp(logp) * (logp - logq);", "d += exp(logp) * (logq - logp);",
     [pins.test_posterior_golden, pins.test_posterior_bernoulli_closed_form]),
    ("lse_drops_max", "double L = mx + log(sum);", "double L = log(sum);",
     [lambda: pins.test_attention_and_lse_vs_library(0)]),
    ("gqa_head_map", "int g = h / G;\n            int i = active_idx",
     "int g = h % Hkv;\n            int i = active_idx",
     [lambda: pins.test_attention_and_lse_vs_library(2)]),
    ("pv_uses_keys", "o[d] += p * wide(vb[(int64_t)n * D + d]);",
     "o[d] += p * wide(kb[(int64_t)n * D + d]);",
     [lambda: pins.test_attention_and_lse_vs_library(0)]),
    ("scale_dropped", "s[n] = scale * dot;", "s[n] = dot;",
     [lambda: pins.test_attention_and_lse_vs_library(1)]),
    ("block_causal_strict", "return slot_n <= slot_i;", "return slot_n < slot_i;",
     [pins.test_visibility_golden]),
    ("group_equal_only", "return group[slot_n] <= group[slot_i];",
     "return group[slot_n] == group[slot_i];", [pins.test_visibility_golden]),
    ("dummy_visible", "if (state[slot_n] == ORA_DUMMY)\n        return 0;", "",
     [pins.test_visibility_golden]),
    ("lock_strict", "locked_out[t] = (uint8_t)(d <= eps &&", "locked_out[t] = (uint8_t)(d < eps &&",
     [pins.test_lock_threshold_is_inclusive]),
    ("lock_ignores_row_flags", "(d <= eps && (flags == NULL || (flags[r] & ORA_ROW_LOCK)) &&",
     "(d <= eps &&", [pins.test_lock_respects_row_flags]),
    ("confidence_gate_ignored", "exp(mx - Lx) >= conf_gate);", "1);", [pins.test_confidence_gate]),
    ("argmax_last", "if ((double)x[v] > mx) {", "if ((double)x[v] >= mx) {",
     [pins.test_posterior_golden]),
    ("colsum_unnormalised", "head_sum += exp(scale * dot - L);", "head_sum += exp(scale * dot);",
     [lambda: pins.test_colsum_vs_explicit_matrix(0, 0)]),
    ("colsum_row_range", "if (i < cs_lo || i >= cs_hi)", "if (i < cs_lo)",
     [lambda: pins.test_colsum_vs_explicit_matrix(0, 0)]),
    ("scatter_wrong_row", "int64_t dst = (((int64_t)b * Hkv + g) * n_cap + pos) * D;",
     "int64_t dst = (((int64_t)b * Hkv + g) * n_cap + j) * D;",
     [pins.test_sparse_equals_full_recompute]),
    ("dynamic_threshold_inclusive", "if (conf[order[t]] > tau && score[order[t]] > thr) {",
     "if (conf[order[t]] > tau && score[order[t]] >= thr) {",
     [pins.test_selection_golden, pins.test_selection_brute_force]),
    ("thresh_conf_inclusive", "if (conf[order[t]] > tau) {", "if (conf[order[t]] >= tau) {",
     [pins.test_selection_golden]),
    ("select_ignores_locks", "if (!locked_in[r] && (flags == NULL",
     "if ((flags == NULL", [pins.test_selection_golden]),
    ("select_ignores_row_flags", "(flags == NULL || (flags[r] & ORA_ROW_SELECT))", "1",
     [pins.test_selection_brute_force]),
    ("entropy_in_bits", "h -= exp(logp) * logp;", "h -= exp(logp) * logp / log(2.0);",
     [pins.test_margin_entropy_vs_library, pins.test_margin_entropy_closed_forms]),
    ("margin_drops_runner_up", "margin[t] = exp(mx - Lx) - (x2 == -INFINITY ? 0.0 : exp(x2 - Lx));",
     "margin[t] = exp(mx - Lx);", [pins.test_margin_entropy_vs_library]),
    ("runner_up_may_be_argmax", "if (v != arg && (double)x[v] > x2)", "if ((double)x[v] > x2)",
     [pins.test_margin_entropy_vs_library]),
    ("entropy_sampler_highest", "neg_entropy[r] = mode == ORA_SEL_TOPK_LOW_ENTROPY ? -entropy[r] : 0.0;",
     "neg_entropy[r] = mode == ORA_SEL_TOPK_LOW_ENTROPY ? entropy[r] : 0.0;",
     [pins.test_selection_golden, pins.test_selection_brute_force]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, checks, tmp_path, monkeypatch):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"mutant_{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"libmutant_{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", str(path),
                    "-o", str(lib), "-lm"], check=True)
    oracle._load()                       # set argtypes on the real library first
    real = oracle._lib
    mutant = ctypes.CDLL(str(lib))
    for fn in ("ora_scatter", "ora_visible", "ora_attn", "ora_colsum", "ora_posterior",
               "ora_select", "ora_num_threads"):
        getattr(mutant, fn).argtypes = getattr(real, fn).argtypes
        getattr(mutant, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(oracle, "_lib", mutant)
    caught = 0
    for check in checks:
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {name}"
