"""Tiled forward recurrence in fp64 -- TEST INFRASTRUCTURE, not the product.

A numpy model of the forward pass the pages describe, used by the CPU tests to
(1) reproduce the intermediate values the pages print for their worked examples
and (2) show that the recurrence reaches the plain definition in
``attention_ref.c``.  It is slow and written for reading, not speed.

Sources (restated, not copied):
  * "6.2 FlashAttention V2 in depth", section 2.2 (query tiles outside, key/value
    tiles inside), section 3.2 (unnormalised accumulator, one division after the
    inner loop), section 5.3 (block classification: fully visible, crossing the
    diagonal, fully masked and skipped) and section 6.1 (the whole forward pass,
    returning O and the per-row statistic L = m + log l).
  * "FlashAttention-2: Where the Second 2x Actually Comes From", section Method
    (the recurrences for m, l and the unnormalised output).
  * "Flash Attention: Memory-Efficient Attention at Scale", section Online softmax
    (running max starts at -inf and running sum at 0; both the sum and the output
    are multiplied by exp(m_old - m_new) when the max grows).

``mistake`` plants one of the slips the pages warn about (or that a port could
make), so that the tests can show they catch it:
  "no_rescale_o"       rescale the running sum but not the running output
  "no_rescale"         rescale neither
  "m_init_zero"        start the running max at 0 instead of -inf
  "normalize_in_loop"  divide the running output by the running sum every step
  "mask_strict"        causal mask keeps key < query instead of key <= query
  "no_diag_mask"       causal: bound the key loop but never mask diagonal tiles
  "lse_log2"           report log2 of the sum instead of the natural log
``form="v1"`` uses the first version's per-step normalised update from section
3.2 of the first page instead, which is algebraically the same result.
"""
from __future__ import annotations

import numpy as np

MISTAKES = ("no_rescale_o", "no_rescale", "m_init_zero", "normalize_in_loop",
            "mask_strict", "no_diag_mask", "lse_log2")


def forward(Q, K, V, Br: int, Bc: int, causal: bool = False, scale: float = 1.0,
            mistake: str | None = None, form: str = "v2", trace: list | None = None):
    """Tiled forward pass of one head.  Q, K, V: [N, d].  Returns (O [N, d], L [N]).

    If ``trace`` is a list, one dict per (query tile, key tile) step is appended
    with the running m, l and unnormalised output after that step.
    """
    if mistake is not None and mistake not in MISTAKES:
        raise ValueError(mistake)
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, d = Q.shape
    O = np.zeros((N, d))
    L = np.zeros(N)
    for i0 in range(0, N, Br):              # query tiles: independent of each other
        rows = np.arange(i0, min(i0 + Br, N))
        Qi = Q[rows]
        m = np.zeros(len(rows)) if mistake == "m_init_zero" else np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), d))      # unnormalised output (normalised in form v1)
        # Causal: key tiles that start after the last row of this query tile are
        # fully masked and never visited.
        kv_end = min(N, i0 + Br) if causal else N
        for j0 in range(0, kv_end, Bc):
            cols = np.arange(j0, min(j0 + Bc, N))
            S = scale * (Qi @ K[cols].T)
            if causal and mistake != "no_diag_mask":
                # Only tiles whose last key lies beyond the first row need the mask.
                if cols[-1] > rows[0]:
                    if mistake == "mask_strict":
                        allowed = cols[None, :] < rows[:, None]
                    else:
                        allowed = cols[None, :] <= rows[:, None]
                    S = np.where(allowed, S, -np.inf)
            m_new = np.maximum(m, S.max(axis=1))
            # A row whose keys so far are all masked keeps m = -inf; it must not
            # produce (-inf) - (-inf).
            m_ref = np.where(np.isneginf(m_new), 0.0, m_new)
            P = np.exp(S - m_ref[:, None])
            alpha = np.exp(m - m_ref)
            if mistake == "no_rescale":
                alpha_l = alpha_o = np.ones_like(alpha)
            elif mistake == "no_rescale_o":
                alpha_l, alpha_o = alpha, np.ones_like(alpha)
            else:
                alpha_l = alpha_o = alpha
            l_new = alpha_l * l + P.sum(axis=1)
            if form == "v1":
                # Keep the output normalised at every step (first version).
                acc = ((l * alpha_o) / l_new)[:, None] * acc + (P @ V[cols]) / l_new[:, None]
            else:
                acc = alpha_o[:, None] * acc + P @ V[cols]
                if mistake == "normalize_in_loop":
                    acc = acc / l_new[:, None]
            m, l = m_new, l_new
            if trace is not None:
                trace.append({"i0": i0, "j0": j0, "m": m.copy(), "l": l.copy(), "acc": acc.copy()})
        if form == "v1" or mistake == "normalize_in_loop":
            O[rows] = acc
        else:
            O[rows] = acc / l[:, None]
        L[rows] = m + (np.log2(l) if mistake == "lse_log2" else np.log(l))
    return O, L


def online_softmax_row(scores, values, block: int):
    """Online softmax over one row of scalar scores and scalar values.

    Returns (per-block list of (m, scale, l, output so far), final output).  This
    is the one-row exercise in the "Practice" section of the lesson page.
    """
    m, l, acc = -np.inf, 0.0, 0.0
    steps = []
    for s0 in range(0, len(scores), block):
        sb = np.asarray(scores[s0:s0 + block], dtype=np.float64)
        vb = np.asarray(values[s0:s0 + block], dtype=np.float64)
        m_new = max(m, float(sb.max()))
        a = float(np.exp(m - m_new))
        p = np.exp(sb - m_new)
        l = l * a + float(p.sum())
        acc = acc * a + float((p * vb).sum())
        m = m_new
        steps.append((m, a, l, acc / l))
    return steps, acc / l
