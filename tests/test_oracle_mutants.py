"""Plant plausible mistakes in a copy of the C oracle and check that the pins
catch every one (mutation testing of the oracle's pins; CPU only).

Each mutant is a textual edit of oracle/attention_ref.c that must apply exactly
as written; it is compiled with gcc into a temporary directory and every pin of
oracle_pins.py runs against it.  A mutant that passes all pins would mean the
pins cannot tell that mistake from the definition.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "attention_ref.c")

# name -> list of (old text, new text, expected number of occurrences)
MUTANTS = {
    "dropped_scale": [("Sr[c] = t->scale * acc;", "Sr[c] = acc;", 1)],
    "transposed_k": [("acc += qr[u] * kc[u];", "acc += qr[u] * t->k[u * N + c];", 1)],
    "transposed_v": [("orow[u] += p * vc[u];", "orow[u] += p * t->v[u * N + c];", 1)],
    "strict_causal": [("t->causal ? r + 1 : N", "t->causal ? r : N", 3)],
    "exp_sign": [("exp(Sr[c] - m)", "exp(m - Sr[c])", 2)],
    "missing_normalisation": [("Sr[c] = exp(Sr[c] - m) / l;", "Sr[c] = exp(Sr[c] - m);", 1)],
    "lse_without_max": [("t->lse[i] = stat_m[i] + log(stat_l[i]);", "t->lse[i] = log(stat_l[i]);", 1)],
    "lse_log2": [("t->lse[i] = stat_m[i] + log(stat_l[i]);", "t->lse[i] = stat_m[i] + log2(stat_l[i]);", 1)],
    "row_min_not_max": [("m = Sr[c] > m ? Sr[c] : m;", "m = Sr[c] < m ? Sr[c] : m;", 1)],
    "no_max_subtraction": [("double m = -INFINITY;\n    for (int64_t c = 0; c < ncols; ++c) m = Sr[c] > m ? Sr[c] : m;",
                            "double m = 0.0;", 1)],
    "block_local_query_row": [("const double* qr = t->q + r * d;", "const double* qr = t->q + i * d;", 1)],
    "pv_skips_first_key": [("for (int64_t c = 0; c < ncols; ++c) {\n      const double p = Pr[c];",
                            "for (int64_t c = 1; c < ncols; ++c) {\n      const double p = Pr[c];", 1)],
    "head_stride_wrong": [("t->k = k + bh * N * d;", "t->k = k + (bh / 2) * N * d;", 1)],
}


def _build_mutant(tmp_path, name):
    with open(SRC) as f:
        text = f.read()
    for old, new, count in MUTANTS[name]:
        assert text.count(old) == count, f"mutant {name}: pattern found {text.count(old)} times"
        text = text.replace(old, new)
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    out = tmp_path / f"lib_{name}.so"
    oracle.build(str(src), str(out))
    return str(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin catches mutant {name}"
