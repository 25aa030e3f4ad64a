"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every ``pin_*`` function takes the path of an oracle library build and raises
AssertionError when the oracle disagrees with:
  * the values the pages print for their worked examples (tests/golden),
  * closed forms of exact attention on hand-built inputs,
  * a textbook library routine (torch softmax in float64 on the CPU),
  * invariants of the definition (rows of weights sum to one, key order does not
    matter without a mask, a causal row never sees later keys, ...),
  * the independent tiled model in ``oracle/tiled.py``.
The same functions run against deliberately broken oracle builds in
``test_oracle_mutants.py`` to show that each plausible mistake fails a pin.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from oracle import tiled
from golden_io import exp_terms, matrix, read_kv, vector


def _att(lib, q, k, v, causal, scale):
    return oracle.attention_f64(q, k, v, causal, scale, nthreads=2, lib_path=lib)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


# --- Worked example of the "Flash Attention 2" page ------------------------------

def pin_worked_example(lib):
    g = read_kv("fa2_page_worked_example.txt")
    Q, K, V = matrix(g["Q"]), matrix(g["KT"]).T.copy(), matrix(g["V"])
    O, L = _att(lib, Q, K, V, False, 1.0)
    l = np.array([exp_terms(g["l_row0_terms"]), exp_terms(g["l_row1_terms"])])
    acc = np.array([[exp_terms(g["acc_r0c0_terms"]), exp_terms(g["acc_r0c1_terms"])],
                    [exp_terms(g["acc_r1c0_terms"]), exp_terms(g["acc_r1c1_terms"])]])
    m = vector(g["m_step3"])
    _close(O[:2], acc / l[:, None], 1e-12, "worked example O rows 0-1 vs closed forms")
    _close(L[:2], m + np.log(l), 1e-12, "worked example L rows 0-1 vs closed forms")
    printed = matrix(g["O_printed"])
    # printed to three decimals; entry (0,0) is the page's arithmetic slip
    for (r, c) in [(0, 1), (1, 0), (1, 1)]:
        assert abs(O[r, c] - printed[r, c]) <= 6e-4, ("printed O", r, c, O[r, c])
    # rows 2..5 are not worked on the page: check them against the definition
    # written out directly (softmax of one row of six scores)
    for r in range(2, 6):
        s = Q[r] @ K.T
        w = np.exp(s - s.max())
        _close(O[r], (w @ V) / w.sum(), 1e-12, f"worked example row {r}")


# --- Practice exercise of the lesson page ----------------------------------------

def _practice_inputs():
    g = read_kv("lesson_practice_online_softmax.txt")
    s = vector(g["scores"])
    vals = vector(g["values"])
    n = len(s)
    Q = np.ones((n, 1))
    K = s[:, None].copy()
    V = vals[:, None].copy()
    return g, Q, K, V


def pin_practice_row(lib):
    g, Q, K, V = _practice_inputs()
    O, L = _att(lib, Q, K, V, False, 1.0)
    final = float(g["final"])
    _close(O[:, 0], np.full(6, final), 6e-7, "practice row, every query row sees all keys")
    steps = g["_steps"]
    m_last, l_last = float(steps[-1][1]), float(steps[-1][3])
    _close(L, np.full(6, m_last + math.log(l_last)), 1e-4, "practice row logsumexp")


def pin_practice_row_causal(lib):
    """With a causal mask, query row 2b+1 sees exactly the keys of blocks 0..b."""
    g, Q, K, V = _practice_inputs()
    O, L = _att(lib, Q, K, V, True, 1.0)
    for st in g["_steps"]:
        b, m, l, out = int(st[0]), float(st[1]), float(st[3]), float(st[4])
        r = 2 * b + 1
        assert abs(O[r, 0] - out) <= 6e-4, ("practice causal O", r, O[r, 0], out)
        assert abs(L[r] - (m + math.log(l))) <= 1e-4, ("practice causal L", r, L[r])
    # row 0 sees only key 0
    _close(O[0], V[0], 0.0, "causal row 0")
    _close(L[:1], Q[0] @ K[0], 0.0, "causal row 0 logsumexp")


# --- Tiled example of the lesson page ---------------------------------------------

def pin_lesson_tiled_vs_standard(lib):
    g = read_kv("lesson_tiled_vs_standard.txt")
    n, d, block = int(g["n"]), int(g["d"]), int(g["block"])
    rs = np.random.RandomState(int(g["seed"]))
    Q, K, V = (rs.randn(n, d) for _ in range(3))
    O, L = _att(lib, Q, K, V, False, 1.0 / math.sqrt(d))
    Ot, Lt = tiled.forward(Q, K, V, Br=n, Bc=block, causal=False, scale=1.0 / math.sqrt(d))
    _close(O, Ot, 1e-13, "lesson tiled vs standard (page prints 3.47e-16)")
    _close(L, Lt, 1e-13, "lesson tiled vs standard, logsumexp")


# --- Closed forms -------------------------------------------------------------------

def pin_closed_form_4x4(lib):
    """Q = K = [I_4 | 0], V = (1..16)/16, multiplier 1: score 1 on the diagonal, 0 elsewhere."""
    Q = np.zeros((4, 6))
    Q[:, :4] = np.eye(4)
    K = Q.copy()
    V = np.arange(1, 25, dtype=np.float64).reshape(4, 6) / 16.0
    e = math.e
    O, L = _att(lib, Q, K, V, False, 1.0)
    for r in range(4):
        want = (e * V[r] + V.sum(axis=0) - V[r]) / (e + 3)
        _close(O[r], want, 1e-15, f"4x4 non-causal row {r}")
        assert abs(L[r] - math.log(e + 3)) <= 1e-15
    O, L = _att(lib, Q, K, V, True, 1.0)
    for r in range(4):
        want = (e * V[r] + V[:r].sum(axis=0)) / (e + r)
        _close(O[r], want, 1e-15, f"4x4 causal row {r}")
        assert abs(L[r] - math.log(e + r)) <= 1e-15, (r, L[r])


def pin_uniform_scores(lib):
    """Multiplier 0: every allowed key has weight 1/|A_r| and L_r = ln |A_r|."""
    rs = np.random.RandomState(3)
    N, d = 37, 5
    Q, K, V = rs.randn(N, d), rs.randn(N, d), rs.randn(N, d)
    O, L = _att(lib, Q, K, V, False, 0.0)
    _close(O, np.broadcast_to(V.mean(axis=0), (N, d)), 1e-14, "scale 0 non-causal")
    _close(L, np.full(N, math.log(N)), 1e-14, "scale 0 non-causal L")
    O, L = _att(lib, Q, K, V, True, 0.0)
    want = np.cumsum(V, axis=0) / np.arange(1, N + 1)[:, None]
    _close(O, want, 1e-14, "scale 0 causal")
    _close(L, np.log(np.arange(1, N + 1)), 1e-14, "scale 0 causal L")


def pin_far_negative_scores(lib):
    """Scores near -2000: exp underflows unless the row max is subtracted."""
    N = 5
    Q = np.full((N, 1), 40.0)
    K = -50.0 - np.arange(N, dtype=np.float64)[:, None] * 0.01
    V = np.arange(N, dtype=np.float64)[:, None] + 1.0
    O, L = _att(lib, Q, K, V, False, 1.0)
    s = (Q[0, 0] * K[:, 0])
    w = np.exp(s - s.max())
    _close(O[:, 0], np.full(N, (w @ V[:, 0]) / w.sum()), 1e-12, "far-negative scores O")
    _close(L, np.full(N, s.max() + math.log(w.sum())), 1e-9, "far-negative scores L")


# --- Library routine ----------------------------------------------------------------

def _torch_reference(q, k, v, causal, scale):
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    s = scale * torch.matmul(qt, kt.transpose(-1, -2).contiguous())
    if causal:
        n = s.shape[-1]
        mask = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
        s = s.masked_fill(mask, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vt)
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


def pin_library_softmax(lib):
    rs = np.random.RandomState(11)
    for (B, H, N, d, causal, scale) in [(2, 3, 37, 5, False, 0.3), (1, 2, 100, 8, True, 0.7),
                                        (1, 1, 130, 3, False, -0.5), (2, 1, 65, 16, True, 0.25)]:
        q, k, v = (rs.randn(B, H, N, d) for _ in range(3))
        O, L = _att(lib, q, k, v, causal, scale)
        Ot, Lt = _torch_reference(q, k, v, causal, scale)
        _close(O, Ot, 1e-12, f"vs torch float64 {(B, H, N, d, causal)}")
        _close(L, Lt, 1e-12, f"vs torch float64 L {(B, H, N, d, causal)}")


# --- Invariants ---------------------------------------------------------------------

def pin_invariants(lib):
    rs = np.random.RandomState(5)
    N, d = 23, 24
    Q, K = rs.randn(N, d), rs.randn(N, d)
    # weights sum to one: V = identity exposes the weights themselves
    for causal in (False, True):
        O, _ = _att(lib, Q, K, np.eye(N, d), causal, 0.4)
        P = O[:, :N]
        _close(P.sum(axis=1), np.ones(N), 1e-14, "weights sum to 1")
        assert np.all(P >= 0)
        if causal:
            assert np.all(np.triu(P, 1) == 0.0), "causal weights above the diagonal"
    # identical V rows come back unchanged
    vrow = rs.randn(d)
    O, _ = _att(lib, Q, K, np.tile(vrow, (N, 1)), False, 0.4)
    _close(O, np.tile(vrow, (N, 1)), 1e-14, "identical V rows")
    # key permutation without a mask
    V = rs.randn(N, d)
    O, L = _att(lib, Q, K, V, False, 0.4)
    perm = rs.permutation(N)
    O2, L2 = _att(lib, Q, K[perm], V[perm], False, 0.4)
    _close(O2, O, 1e-13, "key permutation O")
    _close(L2, L, 1e-13, "key permutation L")
    # causal: a row does not depend on later keys
    O, L = _att(lib, Q, K, V, True, 0.4)
    K2, V2 = K.copy(), V.copy()
    K2[12:] = rs.randn(N - 12, d)
    V2[12:] = rs.randn(N - 12, d)
    O3, L3 = _att(lib, Q, K2, V2, True, 0.4)
    _close(O3[:12], O[:12], 0.0, "future independence O")
    _close(L3[:12], L[:12], 0.0, "future independence L")
    assert np.max(np.abs(O3[12:] - O[12:])) > 1e-3
    # adding u to every key row shifts L by scale*q.u and leaves O alone
    u = rs.randn(d)
    O4, L4 = _att(lib, Q, K + u, V, True, 0.4)
    _close(O4, O, 1e-12, "key shift O")
    _close(L4, L + 0.4 * (Q @ u), 1e-12, "key shift L")
    # (b, h) slices are independent
    q, k, v = (rs.randn(2, 3, 9, 4) for _ in range(3))
    O, L = _att(lib, q, k, v, True, 0.5)
    for b in range(2):
        for h in range(3):
            Os, Ls = _att(lib, q[b, h], k[b, h], v[b, h], True, 0.5)
            _close(O[b, h], Os, 0.0, "(b,h) slice O")
            _close(L[b, h], Ls, 0.0, "(b,h) slice L")


def pin_rows_api(lib):
    rs = np.random.RandomState(9)
    N, d = 150, 7
    Q, K, V = rs.randn(N, d), rs.randn(N, d), rs.randn(N, d)
    rows = np.array([0, 1, 63, 64, 65, 149, 100, 7])
    for causal in (False, True):
        O, L = _att(lib, Q, K, V, causal, 0.3)
        Or, Lr = oracle.attention_rows_f64(Q, K, V, rows, causal, 0.3, nthreads=2, lib_path=lib)
        _close(Or, O[rows], 0.0, "rows API O")
        _close(Lr, L[rows], 0.0, "rows API L")


def pin_tiled_model_agrees(lib):
    rs = np.random.RandomState(21)
    for (N, d, Br, Bc, causal) in [(70, 8, 16, 32, True), (70, 8, 32, 16, True), (33, 4, 8, 8, False),
                                  (129, 16, 64, 32, True), (5, 3, 4, 2, True)]:
        Q, K, V = rs.randn(N, d), rs.randn(N, d), rs.randn(N, d)
        O, L = _att(lib, Q, K, V, causal, 0.6)
        Ot, Lt = tiled.forward(Q, K, V, Br, Bc, causal=causal, scale=0.6)
        _close(Ot, O, 1e-12, f"tiled vs oracle {(N, d, Br, Bc, causal)}")
        _close(Lt, L, 1e-12, f"tiled vs oracle L {(N, d, Br, Bc, causal)}")


PINS = [pin_worked_example, pin_practice_row, pin_practice_row_causal, pin_lesson_tiled_vs_standard,
        pin_closed_form_4x4, pin_uniform_scores, pin_far_negative_scores, pin_library_softmax,
        pin_invariants, pin_rows_api, pin_tiled_model_agrees]
