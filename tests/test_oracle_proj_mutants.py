"""Each plausible mistake planted in a copy of the projection oracle is caught by a pin
(as test_oracle_mutants.py does for the forward oracle).  CPU only."""
import os

import pytest

import oracle
from oracle_proj_pins import PINS

MUTANTS = {
    "head_offset_dropped": ("const uint16_t* wh = w + (size_t)h * C * D;", "const uint16_t* wh = w;"),
    "rq_uses_wq_rows": ("rq[o * dk + j] = oracle_bf16_round(dot(xr, wh + (size_t)(dk + j) * D, D));",
                        "rq[o * dk + j] = oracle_bf16_round(dot(xr, wh + (size_t)j * D, D));"),
    "v_block_offset": ("v[o * d + j] = oracle_bf16_round(dot(xr, wh + (size_t)(2 * dk + j) * D, D));",
                       "v[o * d + j] = oracle_bf16_round(dot(xr, wh + (size_t)(dk + j) * D, D));"),
    "alpha_bias_dropped": ("+ bias[2 * h];", "+ 0.0 * bias[2 * h];"),
    "beta_uses_alpha_bias": ("+ bias[2 * h + 1];", "+ bias[2 * h];"),
    "sigmoid_sign": ("alpha[o] = (float)(1.0 / (1.0 + exp(-za)));", "alpha[o] = (float)(1.0 / (1.0 + exp(za)));"),
    "sum_truncated": ("wq[o * dk + j] = oracle_bf16_round(dot(xr, wh + (size_t)j * D, D));",
                      "wq[o * dk + j] = oracle_bf16_round(trunc(dot(xr, wh + (size_t)j * D, D) * 256.0) / 256.0);"),
    "last_term_dropped": ("for (int k = 0; k < D; ++k)\n        s += bf(xr[k]) * bf(wr[k]);",
                          "for (int k = 0; k + 1 < D; ++k)\n        s += bf(xr[k]) * bf(wr[k]);"),
    "broadcast_one_copy": ("for (int b = 0; b < B; ++b)\n        memcpy(", "for (int b = 0; b < 1; ++b)\n        memcpy("),
}
DIAG_MUTANTS = {
    "bucket_from_second_half": ("acc[(long)nw * K / N] += wt_w[r * W + i];", "acc[(long)(nw % K)] += wt_w[r * W + i];"),
    "writes_not_cumulative": ("                for (int k = 0; k < K; ++k)\n                    cur[k] = 0.0;",
                              "                for (int k = 0; k < K; ++k)\n                    cur[k] = acc[k] = 0.0;"),
    "read_with_write_weights": ("cur[(long)nr * K / N] += wt_r[r * W + i];", "cur[(long)nr * K / N] += wt_w[r * W + i];"),
    "own_token_excluded": ("if (a <= q) {", "if (a < q) {"),
    "overlap_read_weight_dropped": ("s += (double)wt_w[ra * W + i] * wt_r[rq * W + j];", "s += (double)wt_w[ra * W + i];"),
}


def _build_diag(name, old, new):
    src = open(oracle.DIAG_SRC).read()
    assert src.count(old) == 1, f"mutant {name}: the text to change must occur exactly once"
    d = os.path.join(oracle.HERE, "_build")
    os.makedirs(d, exist_ok=True)
    path = os.path.join(d, f"diag_mutant_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    out = os.path.join(d, f"libdiag_mutant_{name}.so")
    import subprocess
    subprocess.run(["gcc", *oracle.CFLAGS, "-Wno-unused-variable", "-I", oracle.HERE, oracle.PROJ_SRC, path, oracle.SRC,
                    "-o", out, "-lm"], check=True)
    return out


@pytest.mark.parametrize("name", sorted(DIAG_MUTANTS))
def test_diag_mutant_is_caught(name):
    assert _caught(oracle.ProjOracle(_build_diag(name, *DIAG_MUTANTS[name]))), f"no pin catches {name!r}"


def _build(name, old, new):
    src = open(oracle.PROJ_SRC).read()
    if old is not None:
        assert src.count(old) == 1, f"mutant {name}: the text to change must occur exactly once"
        src = src.replace(old, new)
    d = os.path.join(oracle.HERE, "_build")
    os.makedirs(d, exist_ok=True)
    path = os.path.join(d, f"proj_mutant_{name}.c")
    with open(path, "w") as f:
        f.write(src)
    return oracle.build_proj(src=path, out=os.path.join(d, f"libproj_mutant_{name}.so"),
                             extra_flags=["-Wno-unused-variable", "-Wno-unused-parameter"])


def _caught(p):
    caught = []
    for pin in PINS:
        try:
            pin(p)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    return caught


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_proj_mutant_is_caught(name):
    assert _caught(oracle.ProjOracle(_build(name, *MUTANTS[name]))), f"no pin catches {name!r}"


def test_unchanged_copy_passes_every_pin():
    assert _caught(oracle.ProjOracle(_build("unchanged", None, None))) == []
