"""Pins of the general-mask oracle against the plain oracle (itself pinned to the
pages in ``oracle_pins.py``) on slices of the same problem, and closed forms.

Each mask admits, for query r, a set of keys whose attention can be written as
plain attention over a slice or a subsequence:
  * a window [r - wl, r + wr] is plain attention over that slice of keys,
  * documents (segment ids) are plain attention over each document's positions,
  * a prefix visible to every query, under a causal mask, is plain attention over
    the prefix for the prefix's rows and plain causal attention for later rows,
so each is checked against the plain oracle called on those slices.
``test_oracle_mask_mutants.py`` runs the same functions against broken builds.
"""
from __future__ import annotations

import numpy as np

import oracle


def _mask(lib, q, k, v, scale, **kw):
    return oracle.attention_masked_f64(q, k, v, scale, nthreads=2, lib_path=lib, **kw)


def _plain(lib, q, k, v, causal, scale):
    return oracle.attention_f64(q, k, v, causal, scale, nthreads=2, lib_path=lib)


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert np.all(np.isfinite(a)), f"{what}: non-finite"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def _inputs(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) for _ in range(3)]


def pin_no_mask_is_plain(lib):
    q, k, v = _inputs(2, 2, 23, 5, 1)
    for causal in (False, True):
        o, l = _mask(lib, q, k, v, 0.4, causal=causal)
        po, pl = _plain(lib, q, k, v, causal, 0.4)
        _close(o, po, 1e-13, f"no mask O (causal={causal})")
        _close(l, pl, 1e-13, f"no mask L (causal={causal})")


def pin_zero_window(lib):
    q, k, v = _inputs(1, 2, 17, 4, 2)
    o, l = _mask(lib, q, k, v, 0.7, window_left=0, window_right=0)
    _close(o, v, 1e-15, "window 0: O = V")
    _close(l, 0.7 * np.sum(q * k, axis=-1), 1e-13, "window 0: L = scale q.k")


def pin_window_is_plain_on_slices(lib):
    N = 29
    q, k, v = _inputs(1, 2, N, 4, 3)
    for wl, wr in ((5, 0), (3, 4), (0, 6), (8, -1), (-1, 2)):
        o, l = _mask(lib, q, k, v, 0.6, window_left=wl, window_right=wr)
        for r in range(N):
            lo = 0 if wl < 0 else max(0, r - wl)
            hi = N - 1 if wr < 0 else min(N - 1, r + wr)
            # plain attention of query r over the window's keys (every row of the
            # slice holds q_r; row 0 is read)
            qq = q[:, :, lo:hi + 1].copy()
            qq[:, :, :] = q[:, :, r:r + 1]
            so, sl = _plain(lib, qq, k[:, :, lo:hi + 1], v[:, :, lo:hi + 1], False, 0.6)
            _close(o[:, :, r], so[:, :, 0], 1e-13, f"window ({wl},{wr}) row {r} O")
            _close(l[:, :, r], sl[:, :, 0], 1e-13, f"window ({wl},{wr}) row {r} L")


def pin_segments_are_plain_per_document(lib):
    N = 31
    q, k, v = _inputs(2, 2, N, 4, 4)
    seg = np.zeros((2, N), dtype=np.int32)
    seg[0] = np.repeat([0, 1, 2, 3], [7, 1, 13, 10])
    seg[1] = np.arange(N) % 3  # interleaved documents
    for causal in (False, True):
        o, l = _mask(lib, q, k, v, 0.5, segment_ids=seg, causal=causal)
        for b in range(2):
            for s_id in np.unique(seg[b]):
                idx = np.nonzero(seg[b] == s_id)[0]
                po, pl = _plain(lib, q[b:b + 1][:, :, idx], k[b:b + 1][:, :, idx], v[b:b + 1][:, :, idx],
                                causal, 0.5)
                _close(o[b:b + 1][:, :, idx], po, 1e-13, f"segment {s_id} of batch {b} O (causal={causal})")
                _close(l[b:b + 1][:, :, idx], pl, 1e-13, f"segment {s_id} of batch {b} L (causal={causal})")


def pin_prefix(lib):
    N = 26
    q, k, v = _inputs(1, 2, N, 4, 5)
    for P in (0, 1, 9, N, N + 5):
        o, l = _mask(lib, q, k, v, 0.45, prefix=P, causal=True)
        pc_o, pc_l = _plain(lib, q, k, v, True, 0.45)
        m = min(P, N)
        if m > 0:
            pp_o, pp_l = _plain(lib, q[:, :, :m], k[:, :, :m], v[:, :, :m], False, 0.45)
            _close(o[:, :, :m], pp_o, 1e-13, f"prefix {P}: prefix rows O")
            _close(l[:, :, :m], pp_l, 1e-13, f"prefix {P}: prefix rows L")
        if m < N:
            _close(o[:, :, max(m, 1):], pc_o[:, :, max(m, 1):], 1e-13, f"prefix {P}: later rows O")
            _close(l[:, :, max(m, 1):], pc_l[:, :, max(m, 1):], 1e-13, f"prefix {P}: later rows L")


def pin_prefix_inside_a_document(lib):
    """A prefix lies inside the first document; other documents never see it."""
    N, P, split = 30, 5, 12
    q, k, v = _inputs(1, 2, N, 4, 6)
    seg = np.array([[0] * split + [1] * (N - split)], dtype=np.int32)
    o, l = _mask(lib, q, k, v, 0.5, prefix=P, segment_ids=seg, causal=True)
    pp_o, pp_l = _plain(lib, q[:, :, :P], k[:, :, :P], v[:, :, :P], False, 0.5)
    _close(o[:, :, :P], pp_o, 1e-13, "prefix rows of document 0")
    d0_o, d0_l = _plain(lib, q[:, :, :split], k[:, :, :split], v[:, :, :split], True, 0.5)
    _close(o[:, :, P:split], d0_o[:, :, P:], 1e-13, "later rows of document 0")
    d1_o, d1_l = _plain(lib, q[:, :, split:], k[:, :, split:], v[:, :, split:], True, 0.5)
    _close(o[:, :, split:], d1_o, 1e-13, "document 1 (no prefix)")
    _close(l[:, :, split:], d1_l, 1e-13, "document 1 L")


MASK_PINS = [pin_no_mask_is_plain, pin_zero_window, pin_window_is_plain_on_slices,
             pin_segments_are_plain_per_document, pin_prefix, pin_prefix_inside_a_document]
