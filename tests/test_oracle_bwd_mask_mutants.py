"""Plant plausible mistakes in the masked gradient oracle's source and check
that at least one pin of oracle_bwd_mask_pins.py fails for each."""
import os

import pytest

import oracle
from oracle_bwd_mask_pins import BWD_MASK_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "attention_bwd_mask_ref.c")

# name -> list of (old text, new text, expected number of occurrences)
MUTANTS = {
    "no_prefix": [("  if (c < t->prefix) return 1;\n", "", 1)],
    "prefix_inclusive": [("if (c < t->prefix) return 1;", "if (c <= t->prefix) return 1;", 1)],
    "window_left_sign": [("c < r - t->wl", "c < r + t->wl", 1)],
    "window_right_strict": [("c > r + t->wr", "c >= r + t->wr", 1)],
    "segments_ignored": [("  if (t->seg && t->seg[c] != t->seg[r]) return 0;\n", "", 1)],
    "segment_batch_wrong": [("t->seg = seg ? seg + (bh / H) * N : NULL;", "t->seg = seg ? seg + (bh % H) * N : NULL;", 1)],
    "masked_keys_in_sum": [("    for (int64_t c = 0; c < N; ++c)\n      if (bwdm_allowed(t, r, c)) l += exp(p[c] - m);",
                            "    for (int64_t c = 0; c < N; ++c) l += exp(bwdm_allowed(t, r, c) ? p[c] - m : 0.0);", 1)],
    "delta_sign": [("const double ds = p[c] * (dp[c] - D);", "const double ds = p[c] * (dp[c] + D);", 1)],
    "dk_unscaled": [("dkc[u] += t->scale * ds * qr[u];", "dkc[u] += ds * qr[u];", 1)],
    "dv_uses_ds": [("dvc[u] += p[c] * gr[u];", "dvc[u] += ds * gr[u];", 1)],
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
    oracle.build(out=str(out), bwd_mask_src=str(src))
    return str(out)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mask_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    caught = []
    for pin in BWD_MASK_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"no pin catches mutant {name}"
