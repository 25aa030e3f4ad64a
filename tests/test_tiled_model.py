"""The test-only tiled model against the intermediate values the pages print,
and the planted mistakes the pages warn about against the oracle."""
import math

import numpy as np
import pytest

import oracle
from oracle import tiled
from golden_io import exp_terms, matrix, read_kv, vector


def test_practice_trace_matches_printed():
    g = read_kv("lesson_practice_online_softmax.txt")
    scores, values = vector(g["scores"]), vector(g["values"])
    steps, final = tiled.online_softmax_row(scores, values, int(g["block"]))
    printed = g["_steps"]
    assert len(steps) == len(printed)
    for (m, a, l, out), p in zip(steps, printed):
        assert m == float(p[1])
        assert abs(a - float(p[2])) <= 5e-4
        assert abs(l - float(p[3])) <= 5e-5
        assert abs(out - float(p[4])) <= 5e-4
    assert abs(final - float(g["final"])) <= 5e-7


@pytest.mark.parametrize("block", [1, 2, 3, 4, 6])
def test_practice_block_size_does_not_change_result(block):
    g = read_kv("lesson_practice_online_softmax.txt")
    _, final = tiled.online_softmax_row(vector(g["scores"]), vector(g["values"]), block)
    assert abs(final - float(g["final"])) <= 5e-7


def test_worked_example_trace_matches_page():
    g = read_kv("fa2_page_worked_example.txt")
    Q, K, V = matrix(g["Q"]), matrix(g["KT"]).T.copy(), matrix(g["V"])
    trace = []
    O, L = tiled.forward(Q, K, V, Br=2, Bc=2, causal=False, scale=1.0, trace=trace)
    first = [t for t in trace if t["i0"] == 0]
    assert len(first) == 3
    for t, key in zip(first, ["m_step1", "m_step2", "m_step3"]):
        np.testing.assert_array_equal(t["m"], vector(g[key]))
    E = math.exp
    # after step 1 the page gives the sums and outputs in closed form
    np.testing.assert_allclose(first[0]["l"], [1 + E(-7), 1 + E(-27)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(first[0]["acc"], [[3 + E(-7), 2 * E(-7)], [3 * E(-27) + 1, 2]],
                               rtol=0, atol=1e-15)
    # after step 2
    np.testing.assert_allclose(first[1]["l"], [1 + E(-3) + E(-10) + E(-11), 1 + E(-3) + E(-18) + E(-27)],
                               rtol=0, atol=1e-15)
    np.testing.assert_allclose(
        first[1]["acc"],
        [[3 * E(-3) + E(-10) - 2 + 5 * E(-11), 2 * E(-10) + 1 - 3 * E(-11)],
         [1 + 3 * E(-27) + 5 * E(-3) - 2 * E(-18), 2 - 3 * E(-3) + E(-18)]], rtol=0, atol=1e-15)
    # after step 3 (final)
    l = [exp_terms(g["l_row0_terms"]), exp_terms(g["l_row1_terms"])]
    acc = [[exp_terms(g["acc_r0c0_terms"]), exp_terms(g["acc_r0c1_terms"])],
           [exp_terms(g["acc_r1c0_terms"]), exp_terms(g["acc_r1c1_terms"])]]
    np.testing.assert_allclose(first[2]["l"], l, rtol=0, atol=1e-15)
    np.testing.assert_allclose(first[2]["acc"], acc, rtol=0, atol=1e-14)
    np.testing.assert_allclose(first[2]["l"], vector(g["l_printed"]), rtol=0, atol=5e-5)
    printed = matrix(g["acc_printed"])
    for (r, c) in [(0, 1), (1, 0), (1, 1)]:
        assert abs(first[2]["acc"][r][c] - printed[r, c]) <= 5e-4
    # the page's decimal for entry (0,0) disagrees with its own closed form
    assert abs(acc[0][0] - printed[0, 0]) > 1e-3


def test_causal_mask_pattern_n4():
    from golden_io import read_matrix_file
    M = read_matrix_file("fa2_page_causal_mask_n4.txt")
    # the tiled model with 1x1 tiles and V = identity exposes the weights; masked
    # entries must be exactly zero and the rest positive
    rs = np.random.RandomState(0)
    Q, K = rs.randn(4, 4), rs.randn(4, 4)
    O, _ = tiled.forward(Q, K, np.eye(4), Br=1, Bc=1, causal=True, scale=1.0)
    np.testing.assert_array_equal(O == 0.0, np.isneginf(M))
    oracle.build()
    Oo, _ = oracle.attention_f64(Q, K, np.eye(4), True, 1.0)
    np.testing.assert_array_equal(Oo == 0.0, np.isneginf(M))


def _case(seed, N, d, far_negative=False):
    rs = np.random.RandomState(seed)
    Q, K, V = rs.randn(N, d), rs.randn(N, d), rs.randn(N, d)
    if far_negative:
        Q = np.abs(Q) + 20.0
        K = -np.abs(K) - 20.0
    return Q, K, V


@pytest.mark.parametrize("form", ["v2", "v1"])
@pytest.mark.parametrize("causal", [False, True])
def test_recurrence_reaches_definition(form, causal):
    oracle.build()
    for (N, d, Br, Bc) in [(70, 8, 16, 32), (70, 8, 32, 16), (33, 5, 8, 8), (9, 2, 4, 4), (1, 3, 4, 4)]:
        Q, K, V = _case(N + d, N, d)
        O, L = oracle.attention_f64(Q, K, V, causal, 0.5)
        Ot, Lt = tiled.forward(Q, K, V, Br, Bc, causal=causal, scale=0.5, form=form)
        np.testing.assert_allclose(Ot, O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(Lt, L, rtol=0, atol=1e-12)


def _fails(mistake):
    """True when the planted mistake makes the model disagree with the oracle on
    at least one of a few small problems."""
    oracle.build()
    for (N, d, Br, Bc, causal, far) in [(70, 8, 16, 32, False, False), (70, 8, 16, 16, True, False),
                                        (12, 4, 4, 4, False, True), (40, 8, 16, 8, True, False)]:
        Q, K, V = _case(7, N, d, far_negative=far)
        scale = 0.5
        O, L = oracle.attention_f64(Q, K, V, causal, scale)
        with np.errstate(all="ignore"):
            Ot, Lt = tiled.forward(Q, K, V, Br, Bc, causal=causal, scale=scale, mistake=mistake)
        if not (np.all(np.isfinite(Ot)) and np.allclose(Ot, O, rtol=0, atol=1e-9)
                and np.allclose(Lt, L, rtol=0, atol=1e-9)):
            return True
    return False


@pytest.mark.parametrize("mistake", tiled.MISTAKES)
def test_each_planted_mistake_is_caught(mistake):
    assert _fails(mistake), f"planted mistake {mistake!r} went unnoticed"


def test_unplanted_model_passes_the_same_checks():
    assert not _fails(None)
