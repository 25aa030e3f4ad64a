"""Plant plausible mistakes in the gradient oracle's source and check that at
least one pin of oracle_bwd_pins.py fails for each: the pins would notice such
a slip in the real oracle."""
import os

import pytest

import oracle
from oracle_bwd_pins import BWD_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "attention_bwd_ref.c")

# name -> list of (old text, new text, expected number of occurrences)
MUTANTS = {
    "no_delta": [("dPr[c] = Pr[c] * (dPr[c] - D);", "dPr[c] = Pr[c] * dPr[c];", 1)],
    "delta_sign": [("dPr[c] = Pr[c] * (dPr[c] - D);", "dPr[c] = Pr[c] * (dPr[c] + D);", 1)],
    "dk_unscaled": [("dkc[u] += t->scale * ds * qr[u];", "dkc[u] += ds * qr[u];", 1)],
    "dq_unscaled": [("dqr[u] += t->scale * ds * kc[u];", "dqr[u] += ds * kc[u];", 1)],
    "dq_uses_v": [("dqr[u] += t->scale * ds * kc[u];", "dqr[u] += t->scale * ds * t->v[c * d + u];", 1)],
    "dk_uses_dout": [("dkc[u] += t->scale * ds * qr[u];", "dkc[u] += t->scale * ds * gr[u];", 1)],
    "dv_uses_ds": [("dvc[u] += p * gr[u];", "dvc[u] += ds * gr[u];", 1)],
    "dp_uses_k": [("const double* vc = t->v + c * d;", "const double* vc = t->k + c * d;", 1)],
    "dv_uses_q": [("dvc[u] += p * gr[u];", "dvc[u] += p * qr[u];", 1)],
    "strict_causal": [("t->causal ? r + 1 : N", "t->causal ? r : N", 1)],
    "no_max_subtraction": [("for (int64_t c = 0; c < ncols; ++c) l += exp(Pr[c] - m);",
                            "m = 0.0;\n      for (int64_t c = 0; c < ncols; ++c) l += exp(Pr[c] - m);", 1),
                           ],
    "unnormalised_p": [("Pr[c] = exp(Pr[c] - m) / l;", "Pr[c] = exp(Pr[c] - m);", 1)],
    "head_stride_wrong": [("t->dout = dout + off;", "t->dout = dout + (bh / 2) * N * d;", 1)],
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
    oracle.build(out=str(out), bwd_src=str(src))
    return str(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    caught = []
    for pin in BWD_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin catches mutant {name}"
