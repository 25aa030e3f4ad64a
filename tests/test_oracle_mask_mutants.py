"""Plant plausible mistakes in the general-mask oracle's source and check that
at least one pin of oracle_mask_pins.py fails for each."""
import os

import pytest

import oracle
from oracle_mask_pins import MASK_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "attention_mask_ref.c")

MUTANTS = {
    "window_left_off_by_one": [("if (t->wl >= 0 && c < r - t->wl) return 0;",
                                "if (t->wl >= 0 && c <= r - t->wl) return 0;", 1)],
    "window_right_off_by_one": [("if (t->wr >= 0 && c > r + t->wr) return 0;",
                                 "if (t->wr >= 0 && c >= r + t->wr) return 0;", 1)],
    "window_right_ignored": [("if (t->wr >= 0 && c > r + t->wr) return 0;", "", 1)],
    "prefix_ignored": [("if (c < t->prefix) return 1;", "", 1)],
    "prefix_inclusive": [("if (c < t->prefix) return 1;", "if (c <= t->prefix) return 1;", 1)],
    "prefix_before_segments": [("  if (t->seg && t->seg[c] != t->seg[r]) return 0;\n  if (c < t->prefix) return 1;",
                                "  if (c < t->prefix) return 1;\n  if (t->seg && t->seg[c] != t->seg[r]) return 0;", 1)],
    "segments_ignored": [("if (t->seg && t->seg[c] != t->seg[r]) return 0;", "", 1)],
    "segments_of_batch_0": [("t->seg = seg ? seg + b * N : NULL;", "t->seg = seg ? seg : NULL;", 1)],
    "lse_without_max": [("t->lse[r] = m + log(l);", "t->lse[r] = log(l);", 1)],
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
    oracle.build(out=str(out), mask_src=str(src))
    return str(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mask_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    caught = []
    for pin in MASK_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin catches mutant {name}"
