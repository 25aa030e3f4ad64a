"""Pins of the decode oracle (new query rows against a key/value cache) against
the plain oracle, itself pinned to the pages in ``oracle_pins.py``, and closed
forms.

Decoding Mq new tokens after a cache of len - Mq tokens is, under the causal
flag, the last Mq rows of plain causal self-attention over the len tokens: the
new rows are the last positions of the sequence.  Without the flag every new
row sees all len cached keys, which is plain non-causal attention of those rows
against the len keys.  Rows past a batch's length never matter.
``test_oracle_decode_mutants.py`` runs the same functions against broken builds.
"""
from __future__ import annotations

import numpy as np

import oracle


def _decode(lib, q, k, v, scale, **kw):
    return oracle.attention_decode_f64(q, k, v, scale, nthreads=2, lib_path=lib, **kw)


def _plain(lib, q, k, v, causal, scale):
    return oracle.attention_f64(q, k, v, causal, scale, nthreads=2, lib_path=lib)


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shapes {a.shape} vs {b.shape}"
    same_inf = np.isneginf(a) & np.isneginf(b)
    assert np.all(np.isfinite(a) | same_inf), f"{what}: non-finite"
    err = float(np.max(np.abs(np.where(same_inf, 0.0, a - b)))) if a.size else 0.0
    assert err <= tol, f"{what}: max |diff| {err:.3e} > {tol:.1e}"


def _seq(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, H, N, d)) for _ in range(3)]


def pin_causal_decode_is_last_rows_of_causal_attention(lib):
    """Per batch b with length len_b: decode of Q[len_b - Mq : len_b] against the
    cache equals rows len_b - Mq .. len_b - 1 of plain causal attention over the
    first len_b tokens."""
    B, H, Nk, d = 3, 2, 40, 5
    Q, K, V = _seq(B, H, Nk, d, 1)
    lens = [40, 17, 9]
    for Mq in (1, 3, 9):
        q = np.stack([Q[b, :, lens[b] - Mq:lens[b]] for b in range(B)])
        o, l = _decode(lib, q, K, V, 0.45, seqlens=lens, causal=True)
        for b in range(B):
            n = lens[b]
            po, pl = _plain(lib, Q[b:b + 1, :, :n], K[b:b + 1, :, :n], V[b:b + 1, :, :n], True, 0.45)
            _close(o[b], po[0, :, n - Mq:], 1e-13, f"Mq={Mq} batch {b} O")
            _close(l[b], pl[0, :, n - Mq:], 1e-13, f"Mq={Mq} batch {b} L")


def pin_noncausal_decode_is_plain_over_the_cache(lib):
    """Without the flag every new row sees all len_b keys: plain non-causal
    attention of a sequence whose first Mq rows are the new queries, over the
    len_b cached keys (the other query rows are filler)."""
    B, H, Nk, d = 2, 3, 33, 4
    _, K, V = _seq(B, H, Nk, d, 2)
    Mq = 4
    q = np.random.default_rng(3).standard_normal((B, H, Mq, d))
    lens = [33, 12]
    o, l = _decode(lib, q, K, V, 0.6, seqlens=lens, causal=False)
    for b in range(B):
        n = lens[b]
        qq = np.zeros((1, H, n, d))
        qq[0, :, :Mq] = q[b]
        po, pl = _plain(lib, qq, K[b:b + 1, :, :n], V[b:b + 1, :, :n], False, 0.6)
        _close(o[b], po[0, :, :Mq], 1e-13, f"batch {b} O")
        _close(l[b], pl[0, :, :Mq], 1e-13, f"batch {b} L")


def pin_cache_rows_past_the_length_never_matter(lib):
    B, H, Nk, d = 2, 2, 30, 4
    Q, K, V = _seq(B, H, Nk, d, 4)
    q = Q[:, :, :3]
    lens = [11, 30]
    o1, l1 = _decode(lib, q, K, V, 0.5, seqlens=lens, causal=True)
    K2, V2 = K.copy(), V.copy()
    K2[0, :, 11:] = 1e3
    V2[0, :, 11:] = -7.0
    o2, l2 = _decode(lib, q, K2, V2, 0.5, seqlens=lens, causal=True)
    _close(o1, o2, 0.0, "O with a changed cache tail")
    _close(l1, l2, 0.0, "L with a changed cache tail")
    # no lengths: the whole cache is valid
    o3, l3 = _decode(lib, q, K, V, 0.5, seqlens=None, causal=False)
    o4, l4 = _decode(lib, q, K, V, 0.5, seqlens=[Nk, Nk], causal=False)
    _close(o3, o4, 0.0, "no lengths = full lengths (O)")
    _close(l3, l4, 0.0, "no lengths = full lengths (L)")


def pin_closed_forms(lib):
    """Scale 0: uniform weights over the visible keys, L = log(count).  One
    visible key: O = that value row, L = its score.  No visible key: O = 0,
    L = -inf."""
    B, H, Nk, d = 2, 1, 12, 3
    _, K, V = _seq(B, H, Nk, d, 5)
    q = np.random.default_rng(6).standard_normal((B, H, 4, d))
    o, l = _decode(lib, q, K, V, 0.0, seqlens=[12, 6], causal=True)
    for b, n in enumerate([12, 6]):
        for i in range(4):
            cnt = n - 4 + i + 1
            _close(o[b, 0, i], V[b, 0, :cnt].mean(axis=0), 1e-14, f"scale 0 batch {b} row {i} O")
            _close(l[b, 0, i], np.log(cnt), 1e-14, f"scale 0 batch {b} row {i} L")
    o, l = _decode(lib, q, K, V, 0.8, seqlens=[1, 3], causal=True)
    # batch 0: only key 0, visible to row 3 alone (rows 0-2 sit before the cache start)
    _close(o[0, 0, 3], V[0, 0, 0], 1e-15, "single key O")
    _close(l[0, 0, 3], 0.8 * float(q[0, 0, 3] @ K[0, 0, 0]), 1e-14, "single key L")
    _close(o[0, 0, :3], np.zeros((3, d)), 0.0, "rows before the cache start O")
    assert np.all(np.isneginf(l[0, 0, :3])), "rows before the cache start L"
    # batch 1, length 3: row 1 sees key 0, row 2 keys 0-1, row 3 keys 0-2
    assert np.isneginf(l[1, 0, 0])
    _close(o[1, 0, 1], V[1, 0, 0], 1e-15, "batch 1 row 1 O")
    o, l = _decode(lib, q, K, V, 0.8, seqlens=[0, 5], causal=False)
    _close(o[0], np.zeros_like(o[0]), 0.0, "empty cache O")
    assert np.all(np.isneginf(l[0])), "empty cache L"


DECODE_PINS = [pin_causal_decode_is_last_rows_of_causal_attention, pin_noncausal_decode_is_plain_over_the_cache,
               pin_cache_rows_past_the_length_never_matter, pin_closed_forms]
