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
    "drop_compensation": ("else *sum = st->s + st->c;", "else *sum = st->s;"),
    "kahan_branch": ("if (fabs(st->s) >= fabs(v))", "if (1)"),
    "swapped_branches": ("st->c += (st->s - t) + v;   /* v's", "st->c += (v - t) + st->s;   /* v's"),
    "wrong_sign": ("st->c += (st->s - t) + v;", "st->c += (t - st->s) + v;"),
    "abs_without_fabs": ("st->a += fabs(v);", "st->a += v;"),
    "inf_pair_not_nan": ("if (st->saw_nan || (st->saw_pinf && st->saw_ninf))", "if (st->saw_nan)"),
    "inf_sign_lost": ("if (v > 0) st->saw_pinf = 1; else st->saw_ninf = 1;", "st->saw_pinf = 1;"),
    "skip_last_element": ("for (i = 0; i < n; ++i)\n        nm_add(&st, (double)x[i]);",
                          "for (i = 0; i + 1 < n; ++i)\n        nm_add(&st, (double)x[i]);"),
    "f64_skips_first": ("for (k = 0; k < n; ++k)", "for (k = 1; k < n; ++k)"),
    "int32_accumulator": ("uint64_t s = 0;", "uint32_t s = 0;"),
    "no_sign_extension": ("s += (uint64_t)(int64_t)x[i];", "s += (uint64_t)(uint32_t)x[i];"),
    "max_starts_at_zero": ("float m = -INFINITY;", "float m = 0.0f;"),
    "max_starts_at_x0": ("float m = -INFINITY;", "float m = n ? x[0] : -INFINITY;"),
    "max_nan_wins": ("if (x[i] > m) m = x[i];", "if (!(x[i] <= m)) m = x[i];"),
    "min_starts_at_zero": ("float m = INFINITY;", "float m = 0.0f;"),
    "argmax_last_of_ties": ("(sign > 0 ? x[i] > m : x[i] < m)", "(sign > 0 ? x[i] >= m : x[i] <= m)"),
    "argext_nan_not_skipped": ("        if (isnan(x[i])) continue;\n", ""),
    "mt_chunk_skips_first": ("for (i = 0; i < ch->n; ++i)", "for (i = 1; i < ch->n; ++i)"),
    "mt_drops_corrections": ("        nm_step(&tot, ch[k].st.c);\n", ""),
    "mt_loses_nan": ("        tot.saw_nan |= ch[k].st.saw_nan;\n", ""),
    "mt_loses_abs": ("        tot.a += ch[k].st.a;\n", "        tot.a = ch[k].st.a;\n"),
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
