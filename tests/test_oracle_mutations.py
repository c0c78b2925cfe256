"""Plant plausible mistakes in copies of oracle.c and check the pins catch each.

Every mutant is compiled on the CPU from a text edit of oracle/oracle.c; the
real oracle is never modified. A mutant that passed every pin would mean the
pins cannot tell that mistake from the correct oracle.
"""
import os

import pytest

from oracle import Oracle
from oracle import build as obuild
from oracle_pins import PINS

MUTATIONS = {
    "drop_compensation": ("else *sum = s + c;", "else *sum = s;"),
    "kahan_branch": ("if (fabs(s) >= fabs(v))", "if (1)"),
    "swapped_branches": ("c += (s - t) + v;   /* v's", "c += (v - t) + s;   /* v's"),
    "wrong_sign": ("c += (s - t) + v;", "c += (t - s) + v;"),
    "abs_without_fabs": ("a += fabs(v);", "a += v;"),
    "inf_pair_not_nan": ("if (saw_nan || (saw_pinf && saw_ninf))", "if (saw_nan)"),
    "inf_sign_lost": ("if (v > 0) saw_pinf = 1; else saw_ninf = 1;", "saw_pinf = 1;"),
    "skip_last_element": ("for (i = 0; i < n; ++i) {\n        double v",
                          "for (i = 0; i + 1 < n; ++i) {\n        double v"),
    "int32_accumulator": ("uint64_t s = 0;", "uint32_t s = 0;"),
    "no_sign_extension": ("s += (uint64_t)(int64_t)x[i];", "s += (uint64_t)(uint32_t)x[i];"),
    "max_starts_at_zero": ("float m = -INFINITY;", "float m = 0.0f;"),
    "max_starts_at_x0": ("float m = -INFINITY;", "float m = n ? x[0] : -INFINITY;"),
    "max_nan_wins": ("if (x[i] > m) m = x[i];", "if (!(x[i] <= m)) m = x[i];"),
    "rows_wrong_stride": ("neumaier_f32(x + r * cols, cols,", "neumaier_f32(x + r, cols,"),
    "rows_max_drops_last_col": ("out[r] = oracle_max_f32(x + r * cols, cols);",
                                "out[r] = oracle_max_f32(x + r * cols, cols - (cols > 0));"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation {name} no longer applies to oracle.c"
    mutant_src = tmp_path / f"{name}.c"
    mutant_src.write_text(src.replace(old, new))
    lib = obuild.build(str(mutant_src), str(tmp_path / f"{name}.so"))
    mutant = Oracle(lib)
    caught = []
    for pin_name, pin in PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin_name)
            break
    assert caught, f"no pin fails for the planted mistake {name}"
    assert os.path.exists(obuild.LIB)
