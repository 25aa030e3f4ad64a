"""Pins of the masked gradient oracle against facts that do not come from it.

Every ``pin_*`` function takes the path of an oracle library build and raises
AssertionError when the gradients under a general mask disagree with:
  * a textbook library routine: torch float64 autograd of
    softmax(scale QK^T + B) V with B = 0 on allowed pairs and -inf elsewhere
    (the mask as a score term, "Flash Attention 2", section "Causal masking"),
    the allowed pairs written out here from the mask's definition,
  * central finite differences of the masked forward oracle,
  * the unmasked and causal gradient oracle (pinned in oracle_bwd_pins.py) for
    the masks that reduce to them,
  * closed forms (a zero multiplier makes every allowed weight uniform),
  * invariants (D = rowsum(dO o O); documents do not interact).
``test_oracle_bwd_mask_mutants.py`` runs the same functions against
deliberately broken builds of the masked gradient source.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _bwd(lib, q, k, v, g, scale, **mask):
    return oracle.attention_bwd_masked_f64(q, k, v, g, scale, nthreads=2, lib_path=lib, **mask)


def _close(a, b, tol, what, rel=False):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shapes {a.shape} {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    if rel:
        err /= max(1.0, float(np.max(np.abs(b))))
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def _inputs(shape, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    return [spread * rng.standard_normal(shape) for _ in range(4)]


def allowed_pairs(N, window_left=-1, window_right=-1, prefix=0, segment_ids=None, causal=False):
    """[B or 1, N, N] boolean: key c allowed for query r."""
    r = np.arange(N)[:, None]
    c = np.arange(N)[None, :]
    wr = 0 if causal else window_right
    win = np.ones((N, N), dtype=bool)
    if window_left >= 0:
        win &= c >= r - window_left
    if wr >= 0:
        win &= c <= r + wr
    ok = (c < prefix) | win
    if segment_ids is None:
        return ok[None]
    seg = np.asarray(segment_ids)
    return ok[None] & (seg[:, :, None] == seg[:, None, :])


MASKS = [
    dict(window_left=3, window_right=2),
    dict(window_left=4, causal=True),
    dict(window_left=2, prefix=3, causal=True),
    dict(prefix=4, window_right=1),
    dict(segment_ids="docs"),
    dict(segment_ids="docs", causal=True, prefix=2, window_left=5),
]


def _mask_for(m, B, N, seed=0):
    m = dict(m)
    if m.get("segment_ids") == "docs":
        rng = np.random.default_rng(100 + seed)
        ids = np.zeros((B, N), dtype=np.int32)
        for b in range(B):
            cuts = np.sort(rng.choice(np.arange(1, N), size=3, replace=False))
            for i, cut in enumerate(cuts):
                ids[b, cut:] = i + 1
        m["segment_ids"] = ids
    return m


def pin_library_autograd(lib):
    """torch float64 autograd of the masked attention, at ordinary scores and at
    scores of several hundred."""
    B, H, N, d = 2, 2, 17, 6
    for i, m in enumerate(MASKS):
        for spread in (1.0, 20.0):
            q, k, v, g = _inputs((B, H, N, d), 10 + i, spread)
            g, v = g / spread, v / spread
            scale = 0.4 if spread == 1.0 else 1.0
            mm = _mask_for(m, B, N, i)
            ok = allowed_pairs(N, **mm)  # [B or 1, N, N]
            bias = torch.tensor(np.where(ok, 0.0, -np.inf))[:, None]  # broadcast over heads
            tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
            s = scale * tq @ tk.transpose(-1, -2) + bias
            o = torch.softmax(s, dim=-1) @ tv
            o.backward(torch.tensor(g))
            dq, dk, dv, _ = _bwd(lib, q, k, v, g, scale, **mm)
            what = f"mask {i} spread {spread}"
            _close(dq, tq.grad.numpy(), 1e-11, f"dQ vs torch autograd ({what})", rel=True)
            _close(dk, tk.grad.numpy(), 1e-11, f"dK vs torch autograd ({what})", rel=True)
            _close(dv, tv.grad.numpy(), 1e-11, f"dV vs torch autograd ({what})", rel=True)


def pin_finite_differences(lib):
    """d sum(O o G) / d x by central differences of the masked forward oracle."""
    h = 1e-6
    B, H, N, d = 1, 1, 7, 3
    for i, m in enumerate((MASKS[0], MASKS[2], MASKS[5])):
        q, k, v, g = _inputs((B, H, N, d), 30 + i)
        mm = _mask_for(m, B, N, i)
        scale = 0.8
        dq, dk, dv, _ = _bwd(lib, q, k, v, g, scale, **mm)

        def loss(qq, kk, vv):
            o, _ = oracle.attention_masked_f64(qq, kk, vv, scale, nthreads=1, lib_path=lib, **mm)
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
            _close(grad, num, 2e-7, f"{name} vs finite differences (mask {i})", rel=True)


def pin_reductions(lib):
    """No bound is the unmasked gradient, a right bound of 0 the causal one,
    and a prefix covering every key the unmasked one again."""
    q, k, v, g = _inputs((2, 2, 19, 5), 40)
    scale = 0.55
    for causal, mask in ((False, {}), (True, dict(causal=True)), (True, dict(window_right=0)),
                         (False, dict(prefix=19, window_left=1, window_right=0)),
                         (False, dict(window_left=18, window_right=18))):
        want = oracle.attention_bwd_f64(q, k, v, g, causal, scale, nthreads=2, lib_path=lib)
        got = _bwd(lib, q, k, v, g, scale, **mask)
        for name, a, b in zip(("dQ", "dK", "dV", "D"), got, want):
            _close(a, b, 1e-13, f"{name} with mask {mask} vs the {'causal' if causal else 'unmasked'} oracle")


def pin_uniform_scores(lib):
    """Multiplier 0: every allowed key of row r has weight 1/|A_r|, dQ = dK = 0
    and dV_c = sum over the rows r that allow c of dO_r / |A_r|."""
    B, H, N, d = 1, 1, 11, 4
    q, k, v, g = _inputs((B, H, N, d), 50)
    for i, m in enumerate(MASKS):
        mm = _mask_for(m, B, N, i)
        ok = allowed_pairs(N, **mm)[0]
        dq, dk, dv, delta = _bwd(lib, q, k, v, g, 0.0, **mm)
        assert np.all(dq == 0.0) and np.all(dk == 0.0), f"dQ, dK must vanish at multiplier 0 (mask {i})"
        cnt = ok.sum(axis=1)
        want = (ok / cnt[:, None]).T @ g[0, 0]
        _close(dv[0, 0], want, 1e-13, f"dV closed form at multiplier 0 (mask {i})")
        mean_v = (ok / cnt[:, None]) @ v[0, 0]
        _close(delta[0, 0], np.sum(g[0, 0] * mean_v, axis=1), 1e-13, f"D closed form (mask {i})")


def pin_invariants(lib):
    q, k, v, g = _inputs((2, 2, 23, 5), 60)
    scale = 0.6
    for i, m in enumerate(MASKS):
        mm = _mask_for(m, 2, 23, i)
        dq, dk, dv, delta = _bwd(lib, q, k, v, g, scale, **mm)
        # D = rowsum(P o dP) equals rowsum(dO o O) with O from the masked forward oracle
        o, _ = oracle.attention_masked_f64(q, k, v, scale, nthreads=2, lib_path=lib, **mm)
        _close(delta, np.sum(g * o, axis=-1), 1e-12, f"D = rowsum(dO o O) (mask {i})")
        # rows of dS sum to zero, so the key sum of dK does
        _close(dk.sum(axis=2), np.zeros((2, 2, 5)), 1e-12, f"sum of dK rows (mask {i})")
    # documents do not interact: two documents, each run as a sequence of its own
    # (the second keeps the window; the prefix lies inside the first)
    N, L1 = 23, 9
    seg = np.array([[0] * L1 + [1] * (N - L1)] * 2, dtype=np.int32)
    for mask in (dict(window_left=3, causal=True, prefix=2), dict(window_left=2, window_right=4)):
        got = _bwd(lib, q, k, v, g, scale, segment_ids=seg, **mask)
        a = _bwd(lib, q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], g[:, :, :L1], scale, **mask)
        m2 = dict(mask)
        m2["prefix"] = 0
        b = _bwd(lib, q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], g[:, :, L1:], scale, **m2)
        for name, x, y, z in zip(("dQ", "dK", "dV", "D"), got, a, b):
            _close(x, np.concatenate([y, z], axis=2), 1e-12, f"{name}: documents one at a time ({mask})")


BWD_MASK_PINS = [pin_library_autograd, pin_finite_differences, pin_reductions, pin_uniform_scores, pin_invariants]
