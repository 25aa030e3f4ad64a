"""Plant plausible mistakes in the decode oracle's source and check that at
least one pin of oracle_decode_pins.py fails for each."""
import os

import pytest

import oracle
from oracle_decode_pins import DECODE_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "attention_decode_ref.c")

MUTANTS = {
    "lengths_ignored": [("t->len = seqlens ? seqlens[bh / H] : Nk;", "t->len = Nk;", 1)],
    "lengths_of_batch_0": [("t->len = seqlens ? seqlens[bh / H] : Nk;", "t->len = seqlens ? seqlens[0] : Nk;", 1)],
    "lengths_per_head": [("t->len = seqlens ? seqlens[bh / H] : Nk;", "t->len = seqlens ? seqlens[bh % B] : Nk;", 1)],
    "causal_top_left": [("if (t->causal) last = t->len - t->Mq + i;", "if (t->causal) last = i;", 1)],
    "causal_strict": [("if (t->causal) last = t->len - t->Mq + i;", "if (t->causal) last = t->len - t->Mq + i - 1;", 1)],
    "causal_ignored": [("if (t->causal) last = t->len - t->Mq + i;", "", 1)],
    "last_key_dropped": [("int64_t last = t->len - 1; /* last allowed key */",
                          "int64_t last = t->len - 2; /* last allowed key */", 1)],
    "query_row_stride": [("const double* qi = t->q + i * d;", "const double* qi = t->q;", 1)],
    "lse_without_max": [("t->lse[i] = m + log(l);", "t->lse[i] = log(l);", 1)],
    "empty_row_nan": [("      t->lse[i] = -INFINITY;\n      continue;", "      t->lse[i] = NAN;\n      continue;", 1)],
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
    oracle.build(out=str(out), decode_src=str(src))
    return str(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_decode_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    caught = []
    for pin in DECODE_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin catches mutant {name}"
