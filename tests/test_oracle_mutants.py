"""Pin strength: plausible mistakes planted in copies of the oracle (on the
CPU, in a temporary directory) must each be caught by some pin check."""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "bevpool_oracle.c")

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("dropped_last_point", "for (int64_t t = t_lo; t < t_hi; ++t) {",
     "for (int64_t t = t_lo; t + 1 < t_hi; ++t) {"),
    ("wrong_sign", "a->out[rb * C + c] += term;", "a->out[rb * C + c] -= term;"),
    ("transposed_feat", "load_value(a->feat, a->feat_dtype, rf * C + c)",
     "load_value(a->feat, a->feat_dtype, c * a->n_feat_rows + rf)"),
    ("feat_row_uses_W", "ranks_feat[t] = (int32_t)((p / dhw) * hw + p % hw);",
     "ranks_feat[t] = (int32_t)((p / dhw) * hw + p % W);"),
    ("feat_row_drops_image", "ranks_feat[t] = (int32_t)((p / dhw) * hw + p % hw);",
     "ranks_feat[t] = (int32_t)(p % hw);"),
    ("depth_index_is_row", "double d = load_value(a->depth, a->depth_dtype, rd);",
     "double d = load_value(a->depth, a->depth_dtype, rf);"),
    ("ties_by_descending_p", "if (x->p != y->p) return x->p < y->p ? -1 : 1;",
     "if (x->p != y->p) return x->p < y->p ? 1 : -1;"),
    ("length_off_by_one",
     "interval_lengths[i] = (int32_t)((i + 1 < I ? interval_starts[i + 1] : N) - interval_starts[i]);",
     "interval_lengths[i] = (int32_t)((i + 1 < I ? interval_starts[i + 1] : N) - interval_starts[i] - (i == 0));"),
    ("f16_exponent_bias", "v = ldexp(1024.0 + m, e - 25);", "v = ldexp(1024.0 + m, e - 24);"),
    ("f16_subnormal_scale", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("e4m3_bias", "v = ldexp(8.0 + m, e - 10);", "v = ldexp(8.0 + m, e - 11);"),
    ("e4m3_nan_code", "if (e == 15 && m == 7)", "if (e == 15)"),
    ("fp8_scale_ignored", "return feat_dtype == ORACLE_E4M3 ? feat_scale : 1.0;",
     "return 1.0;"),
    ("first_point_kept_regardless", "if (point_cell[p] >= 0) { keys[k].cell",
     "if (point_cell[p] >= 0 || p == 0) { keys[k].cell"),
    ("segment_skips_last_point", "for (int64_t t = offsets[s]; t < offsets[s + 1]; ++t) {",
     "for (int64_t t = offsets[s]; t + 1 < offsets[s + 1]; ++t) {"),
    ("segment_weight_ignored", "double w = weights ? load_value(weights, w_dtype, t) : 1.0;",
     "double w = 1.0;"),
    ("segment_row_is_point", "double term = w * (load_value(table, t_dtype, r * C + c) * tscale);",
     "double term = w * (load_value(table, t_dtype, (t % n_rows) * C + c) * tscale);"),
]


RUNNER = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins as P
oracle.use_library({so!r})
caught = []
for check in P.ALL_CHECKS:
    try:
        check()
    except (AssertionError, ValueError) as e:
        caught.append(check.__name__)
print("caught by:", caught)
sys.exit(3 if caught else 0)
"""


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    oracle.build(force=False)
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(workdir, f"lib_{name}.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so,
                           path, "-lm"])
    tests = os.path.dirname(os.path.abspath(__file__))
    code = RUNNER.format(root=os.path.dirname(tests), tests=tests, so=so)
    # a child process, so a mutant that corrupts memory is caught by its crash
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    print(name, r.returncode, r.stdout.strip()[-200:])
    assert r.returncode != 0, f"mutant {name} passed every pin check"
