"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case copies oracle/moe_oracle.c, applies one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, a wrong tie or
rounding rule), builds it with gcc into a temporary directory and runs the
pin tests against it in a subprocess.  The pins pass on the real oracle
(tests/test_oracle_pins.py); here each mutant must make at least one fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "bias_dropped": ("l = l + bias[e];", "l = l;"),
    "router_row_index": ("dot_in(w_router, dtype, (size_t)e * H, x, H)",
                         "dot_in(w_router, dtype, (size_t)e, x, H)"),
    "tie_to_higher_id": ("l[e] > l[best]", "l[e] >= l[best]"),
    "gate_renormalised": ("topk_w[(size_t)t * K + k] = (float)p[best];",
                          "topk_w[(size_t)t * K + k] = (float)(p[best] * 2.0);"),
    "silu_sign": ("double silu = ga / (1.0 + exp(-ga));",
                  "double silu = ga / (1.0 + exp(ga));"),
    "gate_up_swapped": ("double silu = ga / (1.0 + exp(-ga));\n            a[(size_t)r * I + i] = (double)(float)(silu * ub);",
                        "double silu = ub / (1.0 + exp(-ub));\n            a[(size_t)r * I + i] = (double)(float)(silu * ga);"),
    "down_transposed": ("dot_in(wd, dtype, (size_t)o * I,", "dot_in(wd, dtype, (size_t)o,"),
    "dispatch_reverse_in_group": ("int row = offsets[s] + fill[s]++;",
                                  "int row = offsets[s + 1] - 1 - fill[s]++;"),
    "replica_hash_drops_k": ("seed ^ (tok * (uint64_t)K + (uint64_t)k)", "seed ^ (tok * (uint64_t)K)"),
    "shared_gate_sign": ("gate[t] = (float)(1.0 / (1.0 + exp(-(double)z)));",
                         "gate[t] = (float)(1.0 / (1.0 + exp((double)z)));"),
    "e4m3_round_half_up": ("long m = lrint((2.0 * f - 1.0) * 8.0);",
                           "long m = (long)floor((2.0 * f - 1.0) * 8.0 + 0.5);"),
    "quant_scale_inverted": ("scale[r] = amax / 448.0f;", "scale[r] = 448.0f / amax;"),
    "shared_term_dropped": ("acc[(size_t)t * H + o] += (double)gs[t] * shsum[(size_t)t * H + o];",
                            "acc[(size_t)t * H + o] += 0.0 * shsum[(size_t)t * H + o];"),
    "splitmix_shift": ("z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;",
                       "z = (z ^ (z >> 28)) * 0x94D049BB133111EBull;"),
    "f16_exponent_bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "group_tie_to_higher_id": ("if (bg < 0 || sc > bs)", "if (bg < 0 || sc >= bs)"),
    "group_score_first_expert": ("                            sc = l[e];", "                            sc = sc;"),
    "group_mask_wrong_group": ("if (!gsel[e / gs])", "if (!gsel[e % G])"),
    "replica_mod_off_by_one": ("(uint64_t)n);", "(uint64_t)(n + 1));"),
    "replica_hash_only_above_two": ("if (n > 1)", "if (n > 2)"),
    "combine_weight_of_next_k": ("acc += (double)topk_w[(size_t)t * K + k] * (double)y[(size_t)r * H + o];",
                                 "acc += (double)topk_w[(size_t)t * K + (k + 1) % K] * (double)y[(size_t)r * H + o];"),
    "expert_input_wrong_token": ("            int t = pair[r] / K;\n            if (d->fp8_dispatch) {",
                                 "            int t = pair[r] % K;\n            if (d->fp8_dispatch) {"),
    "dispatch_offsets_skip_first_slot": ("offsets[s + 1] = offsets[s] + counts[s];",
                                         "offsets[s + 1] = offsets[s] + (s ? counts[s] : 0);"),
    "combine_skips_last_k": ("            for (int k = 0; k < K; ++k) {\n                int r = inv_pos",
                             "            for (int k = 0; k < K - 1; ++k) {\n                int r = inv_pos"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", str(lib), str(mut), "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
