"""Each plausible mistake planted in a copy of the gradient oracle is caught by a pin.

As for the forward oracle (test_oracle_mutants.py): the source of
oracle/sdm_oracle_grad.c is copied, one textual change is made, the copy is
built with the same flags (with the unchanged forward it replays), and the
gradient pins run against it; at least one must fail.  CPU only.
"""
import os

import pytest

import oracle
from oracle_grad_pins import ADDRESS_PINS, SCAN_PINS

MUTANTS = {
    "read_gradient_dropped": (
        "                G[(size_t)m[j] * d + e] += (double)rw[j] * (double)go[e];",
        "                G[(size_t)m[j] * d + e] += 0.0 * (double)rw[j] * (double)go[e];"),
    "read_weight_dropped": ("G[(size_t)m[j] * d + e] += (double)rw[j] * (double)go[e];",
                            "G[(size_t)m[j] * d + e] += (double)go[e];"),
    "decay_dropped_in_state_grad": ("G[(size_t)n[i] * d + e] = a * dx;", "G[(size_t)n[i] * d + e] = dx;"),
    "state_grad_accumulated": ("G[(size_t)n[i] * d + e] = a * dx;", "G[(size_t)n[i] * d + e] += a * dx;"),
    "prediction_grad_sign": ("const double dvhat = -be * ddelta[e];", "const double dvhat = be * ddelta[e];"),
    "prediction_grad_dropped": ("const double dx = gi + (double)w[i] * dvhat;", "const double dx = gi;"),
    "dv_without_beta": ("dv[r * d + e] = be * dd;", "dv[r * d + e] = dd;"),
    "dbeta_uses_prediction": ("db += dd * (ve - yh);", "db += dd * ve;"),
    "dw_drops_delta_term": ("dw += gi * delta[e] + dvhat * x[(size_t)i * d + e];",
                            "dw += dvhat * x[(size_t)i * d + e];"),
    "dw_drops_prediction_term": ("dw += gi * delta[e] + dvhat * x[(size_t)i * d + e];", "dw += gi * delta[e];"),
    "dalpha_uses_decayed": ("da += dx * wlog[((size_t)t * W + i) * d + e];", "da += dx * x[(size_t)i * d + e];"),
    "no_restore": ("                if (kind == 2)\n                    ((double*)work)[at] = old;",
                   "                if (kind == 2)\n                    ((double*)work)[at] = ((double*)work)[at] + 0.0 * old;"),
    "softmax_grad_without_mean": ("const double ds = w[i] * (gw[i] - mean);", "const double ds = w[i] * gw[i];"),
    "softmax_grad_without_weight": ("const double ds = w[i] * (gw[i] - mean);", "const double ds = gw[i] - mean;"),
    "dq_halves_swapped": ("gq[j] += ds * in_value(subkeys, k0, c->in_bf16);",
                          "gq[j] += ds * in_value(subkeys, k1, c->in_bf16);"),
    "dsub_second_half_index": ("const size_t k1 = (((size_t)h * 2 + 1) * S + bb) * dh + j;",
                               "const size_t k1 = (((size_t)h * 2 + 1) * S + a) * dh + j;"),
    "dsub_wrong_query_half": ("dsub[k1] += ds * in_value(q, (size_t)r * dk + dh + j, c->in_bf16);",
                              "dsub[k1] += ds * in_value(q, (size_t)r * dk + j, c->in_bf16);"),
}


def _build(name, old, new):
    src = open(oracle.GRAD_SRC).read()
    if old is not None:
        assert src.count(old) == 1, f"mutant {name}: the text to change must occur exactly once"
        src = src.replace(old, new)
    d = os.path.join(oracle.HERE, "_build")
    os.makedirs(d, exist_ok=True)
    path = os.path.join(d, f"grad_mutant_{name}.c")
    with open(path, "w") as f:
        f.write(src)
    return oracle.build_grad(src=path, out=os.path.join(d, f"libgrad_mutant_{name}.so"),
                             extra_flags=["-Wno-unused-variable", "-Wno-unused-parameter",
                                          "-Wno-unused-but-set-variable"])


def _caught(g):
    caught = []
    o = oracle.get()
    for pin in SCAN_PINS:
        try:
            pin(g)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    for pin in ADDRESS_PINS:
        try:
            pin(g, o)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    return caught


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_grad_mutant_is_caught(name):
    g = oracle.GradOracle(_build(name, *MUTANTS[name]))
    assert _caught(g), f"no pin catches the planted mistake {name!r}"


def test_unchanged_copy_passes_every_pin():
    """The harness itself: an unchanged copy built the same way passes every pin."""
    g = oracle.GradOracle(_build("unchanged", None, None))
    assert _caught(g) == []
