"""Each plausible mistake planted in a copy of the oracle is caught by a pin.

The oracle source is copied, one textual change is made, the copy is built
with the same flags and every pin runs against it; at least one pin must fail.
This shows that the pins constrain the oracle where a slip would matter (a
dropped term, a wrong sign or index, a transposed operand, a wrong order).
CPU only; the mutants live under oracle/_build/ and are never used elsewhere.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    "decay_dropped": ("x[(size_t)i * ne + e] = a * load_state(", "x[(size_t)i * ne + e] = 1.0 * load_state("),
    "beta_dropped": ("delta[e] = be * (", "delta[e] = 1.0 * ("),
    "delta_sign": ("(load_in(v, r * d + e0 + e, c->in_bf16) - vhat)", "(vhat - load_in(v, r * d + e0 + e, c->in_bf16))"),
    "write_weight_dropped": ("x[(size_t)i * ne + e] + (double)w[i] * delta[e]", "x[(size_t)i * ne + e] + delta[e]"),
    "prediction_before_decay": ("vhat += (double)w[i] * x[(size_t)i * ne + e];",
                                "vhat += (double)w[i] * x[(size_t)i * ne + e] / a;"),
    "read_with_write_weights": ("o += (double)rw[j] *", "o += (double)w[j] *"),
    "read_drops_last_slot": ("for (int j = 0; j < W; ++j) {\n                if (m[j] < 0",
                             "for (int j = 0; j + 1 < W; ++j) {\n                if (m[j] < 0"),
    "slot_index_transposed": ("cand[(size_t)i * k + j].i = a[i] * S + b[j];", "cand[(size_t)i * k + j].i = b[j] * S + a[i];"),
    "subkey_tables_swapped": ("(((size_t)h * 2 + half) * S + i) * dh + j", "(((size_t)h * 2 + (1 - half)) * S + i) * dh + j"),
    "query_halves_swapped": ("(size_t)r * c->dk + (size_t)half * dh + j", "(size_t)r * c->dk + (size_t)(1 - half) * dh + j"),
    "second_half_uses_first_list": ("float sum = s1[a[i]] + s2[b[j]];", "float sum = s1[a[i]] + s2[a[j]];"),
    "tie_break_reversed": ("return (a->i > b->i) - (a->i < b->i);", "return (a->i < b->i) - (a->i > b->i);"),
    "order_ascending": ("if (a->v > b->v)\n        return -1;\n    if (a->v < b->v)\n        return 1;",
                        "if (a->v < b->v)\n        return -1;\n    if (a->v > b->v)\n        return 1;"),
    "softmax_unnormalised": ("w[i] = (float)(exp((double)sigma[i] - m) / z);", "w[i] = (float)(exp((double)sigma[i] - m));"),
    "softmax_temperature": ("w[i] = (float)(exp((double)sigma[i] - m) / z);",
                            "w[i] = (float)(exp((double)sigma[i] - m) / z * 0 + exp(0.5 * ((double)sigma[i] - m)) / z);"),
    "bf16_truncates": ("nearbyint(a / q)", "floor(a / q)"),
    "bf16_wrong_width": ("int qexp = e - 8;", "int qexp = e - 9;"),
    "state_rounding_skipped": ("((float*)mem)[i] = (float)x;", "((float*)mem)[i] = (float)(x + x * 0x1p-20);"),
    "score_rounded_twice": ("acc += qj * kj;", "acc = (float)(acc + qj * kj);"),
    "head_ignored_in_subkeys": ("int h = (int)(r % c->H);\n        for (int half", "int h = 0;\n        for (int half"),
    # selection from given scores: the second half read from the first half's row
    "scores_second_half_misplaced": ("const float* s2 = scores + (o * 2 + 1) * S;",
                                     "const float* s2 = scores + (o * 2 + 0) * S;"),
    # selection from given scores: a row's output written at the previous row's place
    "scores_rows_shifted": ("oracle_select(s1, s2, S, c->k, W, idx + o * W, sig)",
                            "oracle_select(s1, s2, S, c->k, W, idx + (o ? o - 1 : o) * W, sig)"),
    # the scan's element slice: v read from the slice's first element instead of its own
    "scan_slice_offset_dropped_for_v": ("(load_in(v, r * d + e0 + e, c->in_bf16) - vhat)",
                                        "(load_in(v, r * d + e, c->in_bf16) - vhat)"),
}


def _build_mutant(name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutant {name}: the text to change must occur exactly once in the oracle"
    d = os.path.join(oracle.HERE, "_build")
    os.makedirs(d, exist_ok=True)
    path = os.path.join(d, f"mutant_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    return oracle.build(src=path, out=os.path.join(d, f"libmutant_{name}.so"),
                        extra_flags=["-Wno-unused-variable", "-Wno-unused-parameter", "-Wno-unused-but-set-variable"])


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    o = oracle.Oracle(_build_mutant(name, old, new))
    caught = []
    for pin in PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
        except ValueError:  # the mutant broke an argument check: also a catch
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
