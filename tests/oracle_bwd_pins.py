"""Pins of the gradient oracle against facts that do not come from it.

Every ``pin_*`` function takes the path of an oracle library build and raises
AssertionError when the gradients disagree with:
  * central finite differences of the forward oracle (itself pinned to the
    pages in ``oracle_pins.py``): the gradient is the derivative of
    sum(O o G) with respect to Q, K and V, element by element,
  * a textbook library routine (torch autograd in float64 on the CPU),
  * closed forms (a zero multiplier makes every weight uniform),
  * invariants of the definition (rows of dS sum to zero, so the rows of dK do;
    shifting every key by one vector changes nothing; a causal row 0 sees only
    key 0) and the identity rowsum(P o dP) = rowsum(dO o O) that
    "6.2 FlashAttention V2 in depth" (section 7.3) uses for D.
``test_oracle_bwd_mutants.py`` runs the same functions against deliberately
broken builds of the gradient source.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _bwd(lib, q, k, v, g, causal, scale):
    return oracle.attention_bwd_f64(q, k, v, g, causal, scale, nthreads=2, lib_path=lib)


def _fwd(lib, q, k, v, causal, scale):
    return oracle.attention_f64(q, k, v, causal, scale, nthreads=2, lib_path=lib)


def _close(a, b, tol, what, rel=False):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    if rel:
        err /= max(1.0, float(np.max(np.abs(b))))
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def _inputs(shape, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    return [spread * rng.standard_normal(shape) for _ in range(4)]


def pin_finite_differences(lib):
    """d sum(O o G) / d x by central differences of the forward oracle."""
    h = 1e-6
    for causal, N, d, scale, seed in ((False, 5, 3, 0.7, 1), (True, 6, 3, 0.9, 2), (True, 4, 2, -0.4, 3)):
        q, k, v, g = _inputs((N, d), seed)
        dq, dk, dv, _ = _bwd(lib, q, k, v, g, causal, scale)

        def loss(qq, kk, vv):
            o, _ = _fwd(lib, qq, kk, vv, causal, scale)
            return float(np.sum(o * g))

        for name, x, grad in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"dQ": (xp, k, v), "dK": (q, xp, v), "dV": (q, k, xp)}[name]
                args_m = {"dQ": (xm, k, v), "dK": (q, xm, v), "dV": (q, k, xm)}[name]
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            _close(grad, num, 2e-7, f"{name} vs finite differences (causal={causal}, N={N})", rel=True)


def pin_library_autograd(lib):
    """torch float64 autograd of softmax(scale QK^T + mask) V, at ordinary
    scores and at scores of several hundred (exp overflows unless the row max
    is taken out first)."""
    for causal, seed, spread in ((False, 5, 1.0), (True, 6, 1.0), (False, 9, 20.0), (True, 10, 20.0)):
        q, k, v, g = _inputs((2, 3, 20, 8), seed, spread)
        g, v = g / spread, v / spread
        scale = 0.35 if spread == 1.0 else 1.0
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        s = scale * tq @ tk.transpose(-1, -2)
        if causal:
            s = s.masked_fill(torch.ones(20, 20, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        o.backward(torch.tensor(g))
        dq, dk, dv, _ = _bwd(lib, q, k, v, g, causal, scale)
        _close(dq, tq.grad.numpy(), 1e-11, f"dQ vs torch autograd (causal={causal}, spread={spread})", rel=True)
        _close(dk, tk.grad.numpy(), 1e-11, f"dK vs torch autograd (causal={causal}, spread={spread})", rel=True)
        _close(dv, tv.grad.numpy(), 1e-11, f"dV vs torch autograd (causal={causal}, spread={spread})", rel=True)


def pin_uniform_scores(lib):
    """Multiplier 0: every allowed key has weight 1/|A_r|, dQ = dK = 0 and
    dV_c = sum over the rows that see key c of dO_r / |A_r|."""
    N, d = 9, 4
    q, k, v, g = _inputs((N, d), 7)
    for causal in (False, True):
        dq, dk, dv, delta = _bwd(lib, q, k, v, g, causal, 0.0)
        assert np.all(dq == 0.0) and np.all(dk == 0.0), "dQ, dK must vanish at multiplier 0"
        counts = np.arange(1, N + 1) if causal else np.full(N, N)
        want = np.zeros((N, d))
        for r in range(N):
            for c in range(counts[r] if causal else N):
                want[c] += g[r] / counts[r]
        _close(dv, want, 1e-13, f"dV closed form at multiplier 0 (causal={causal})")
        mean_v = np.array([v[: counts[r]].mean(0) if causal else v.mean(0) for r in range(N)])
        _close(delta, np.sum(g * mean_v, axis=1), 1e-13, f"D closed form (causal={causal})")


def pin_invariants(lib):
    q, k, v, g = _inputs((2, 2, 33, 5), 8)
    scale = 0.6
    for causal in (False, True):
        dq, dk, dv, delta = _bwd(lib, q, k, v, g, causal, scale)
        # rows of dS sum to zero, so the key-sum of dK = scale dS^T Q vanishes
        _close(dk.sum(axis=2), np.zeros((2, 2, 5)), 1e-12, f"sum of dK rows (causal={causal})")
        # D = rowsum(P o dP) equals rowsum(dO o O) with O from the forward oracle
        o, _ = _fwd(lib, q, k, v, causal, scale)
        _close(delta, np.sum(g * o, axis=-1), 1e-12, f"D = rowsum(dO o O) (causal={causal})")
        # adding one vector to every key row shifts each score row by a constant
        u = np.array([0.3, -1.1, 0.7, 0.2, -0.5])
        dq2, dk2, dv2, _ = _bwd(lib, q, k + u, v, g, causal, scale)
        _close(dq2, dq, 1e-11, f"dQ under a key shift (causal={causal})")
        _close(dk2, dk, 1e-11, f"dK under a key shift (causal={causal})")
        _close(dv2, dv, 1e-12, f"dV under a key shift (causal={causal})")
        # each (b, h) slice is independent
        s_dq, s_dk, s_dv, _ = _bwd(lib, q[1, 0], k[1, 0], v[1, 0], g[1, 0], causal, scale)
        _close(s_dq, dq[1, 0], 0.0, "dQ slice independence")
        _close(s_dk, dk[1, 0], 0.0, "dK slice independence")
        _close(s_dv, dv[1, 0], 0.0, "dV slice independence")
    # causal: row 0 sees only key 0 (weight 1, so dS row 0 is zero and dQ_0 = 0);
    # the last key is seen only by the last row
    dq, dk, dv, _ = _bwd(lib, q[0, 0], k[0, 0], v[0, 0], g[0, 0], True, scale)
    assert np.all(dq[0] == 0.0), "causal dQ row 0 must be zero"
    o, lse = _fwd(lib, q[0, 0], k[0, 0], v[0, 0], True, scale)
    p_last = np.exp(scale * q[0, 0][-1] @ k[0, 0][-1] - lse[-1])
    _close(dv[-1], p_last * g[0, 0][-1], 1e-12, "causal dV of the last key")


BWD_PINS = [pin_finite_differences, pin_library_autograd, pin_uniform_scores, pin_invariants]
