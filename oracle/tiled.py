"""Tiled forward recurrence in fp64 -- TEST INFRASTRUCTURE, not the product.

A numpy model of how the forward pass reaches exact attention block by block,
used by the CPU tests to (1) reproduce the intermediate values the pages print
for their worked examples and (2) show that the recurrence reaches the plain
definition in ``attention_ref.c``.  It is slow and written for reading.

The model is built on one object, the softmax statistics of a set of query rows
over some subset of the keys, ``Partial(m, l, acc)``:
  m   the reference of each row (the largest score seen; -inf before any key),
  l   the sum of exp(s - m) over the keys seen,
  acc the sum of exp(s - m) * v over the keys seen (unnormalised output).
Two partials over disjoint key sets combine exactly by moving both to the larger
reference (``merge``); the result over all keys is acc / l with the per-row
statistic L = m + log l (``finish``).  Folding the key blocks into a running
partial one at a time is the online softmax; the order and the grouping of the
blocks do not change the result.

What the pages fix, and where:
  * the running max, running sum and unnormalised output, each rescaled by
    exp(m_old - m_new) when the max grows, divided by the sum once at the end:
    "6.2 FlashAttention V2 in depth", sections 3.2 and 6.1; "FlashAttention-2:
    Where the Second 2x Actually Comes From", section "Method"; the running max
    starts at -inf and the sum at 0: "Flash Attention: Memory-Efficient
    Attention at Scale", section "Online softmax";
  * the per-block form (each block's own max and sum, then combined) is the one
    the "Flash Attention 2" page writes out; it equals the running-max form;
  * the statistic L = m + log l: "6.2 FlashAttention V2 in depth", section 7.1;
  * query blocks are independent; under a causal mask key blocks past a query
    block's last row are never visited and blocks crossing the diagonal are
    masked element by element: same page, sections 2.2 and 5.3.

``mistake`` plants one of the slips the pages warn about (or that a port could
make), so that the tests can show they catch it:
  "no_rescale_o"       rescale the running sum but not the running output
  "no_rescale"         rescale neither
  "m_init_zero"        start the running max at 0 instead of -inf
  "normalize_in_loop"  divide the running output by the running sum every step
  "mask_strict"        causal mask keeps key < query instead of key <= query
  "no_diag_mask"       causal: bound the key loop but never mask diagonal tiles
  "lse_log2"           report log2 of the sum instead of the natural log
``form="v1"`` keeps the output normalised after every block (the first
version's update, "6.2 FlashAttention V2 in depth", section 3.2), which is
algebraically the same result.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MISTAKES = ("no_rescale_o", "no_rescale", "m_init_zero", "normalize_in_loop",
            "mask_strict", "no_diag_mask", "lse_log2")


@dataclass
class Partial:
    """Softmax statistics of R query rows over a subset of the keys (see the
    module docstring).  ``acc`` is [R, d]; in the normalised form ("v1") it
    holds acc / l instead."""
    m: np.ndarray
    l: np.ndarray
    acc: np.ndarray

    @staticmethod
    def empty(rows: int, d: int, m0: float = -np.inf) -> "Partial":
        return Partial(np.full(rows, m0), np.zeros(rows), np.zeros((rows, d)))


def _finite_ref(m):
    # A row that has seen only masked keys keeps m = -inf; exponents are then
    # taken against 0 so that no (-inf) - (-inf) appears (its weights are 0).
    return np.where(np.isneginf(m), 0.0, m)


def block_partial(S, Vb) -> Partial:
    """The statistics of one block alone: scores S [R, c] (-inf where masked)
    and values Vb [c, d], against the block's own row max."""
    m = S.max(axis=1) if S.shape[1] else np.full(S.shape[0], -np.inf)
    P = np.exp(S - _finite_ref(m)[:, None])
    return Partial(m, P.sum(axis=1), P @ Vb)


def merge(a: Partial, b: Partial, rescale_l: bool = True, rescale_acc: bool = True,
          normalised: bool = False) -> Partial:
    """Combine two partials over disjoint key sets: both move to the larger
    reference, their sums and outputs add.  The flags plant the rescaling slips
    (a factor left out on the running side ``a``); ``normalised`` combines two
    partials whose ``acc`` holds acc / l."""
    m = np.maximum(a.m, b.m)
    ref = _finite_ref(m)
    fa, fb = np.exp(a.m - ref), np.exp(b.m - ref)
    la = fa * a.l if rescale_l else a.l
    l = la + fb * b.l
    if normalised:
        with np.errstate(invalid="ignore", divide="ignore"):
            wa = np.where(l > 0, (fa * a.l) / l, 0.0)
            wb = np.where(l > 0, (fb * b.l) / l, 0.0)
        return Partial(m, l, wa[:, None] * a.acc + wb[:, None] * b.acc)
    acc_a = fa[:, None] * a.acc if rescale_acc else a.acc
    return Partial(m, l, acc_a + fb[:, None] * b.acc)


def finish(p: Partial, log=np.log, normalised: bool = False):
    """Output rows and their statistic L = m + log l."""
    O = p.acc if normalised else p.acc / p.l[:, None]
    return O, p.m + log(p.l)


def _scores(Q, K, rows, cols, causal, scale, mistake):
    """Scaled scores of query rows x key columns; under the causal mask a block
    that crosses the diagonal (its last key beyond its first row) is masked
    element by element."""
    S = scale * (Q[rows] @ K[cols].T)
    if causal and mistake != "no_diag_mask" and cols[-1] > rows[0]:
        keep = (cols[None, :] < rows[:, None]) if mistake == "mask_strict" else (cols[None, :] <= rows[:, None])
        S = np.where(keep, S, -np.inf)
    return S


def forward(Q, K, V, Br: int, Bc: int, causal: bool = False, scale: float = 1.0,
            mistake: str | None = None, form: str = "v2", trace: list | None = None):
    """Tiled forward pass of one head.  Q, K, V: [N, d].  Returns (O [N, d], L [N]).

    If ``trace`` is a list, one dict per (query block, key block) step is
    appended with the running m, l and acc after that step.
    """
    if mistake is not None and mistake not in MISTAKES:
        raise ValueError(mistake)
    Q, K, V = (np.asarray(t, dtype=np.float64) for t in (Q, K, V))
    N, d = Q.shape
    normalised = form == "v1"
    O, L = np.zeros((N, d)), np.zeros(N)
    for i0 in range(0, N, Br):
        rows = np.arange(i0, min(i0 + Br, N))
        run = Partial.empty(len(rows), d, 0.0 if mistake == "m_init_zero" else -np.inf)
        last_key = rows[-1] if causal else N - 1       # later key blocks are never visited
        for j0 in range(0, last_key + 1, Bc):
            cols = np.arange(j0, min(j0 + Bc, N))
            blk = block_partial(_scores(Q, K, rows, cols, causal, scale, mistake), V[cols])
            if normalised:  # a row with no visible key in the block keeps a zero output
                with np.errstate(invalid="ignore", divide="ignore"):
                    blk = Partial(blk.m, blk.l, np.where(blk.l[:, None] > 0, blk.acc / blk.l[:, None], 0.0))
            run = merge(run, blk, rescale_l=mistake != "no_rescale",
                        rescale_acc=mistake not in ("no_rescale", "no_rescale_o"), normalised=normalised)
            if mistake == "normalize_in_loop":
                run = Partial(run.m, run.l, run.acc / run.l[:, None])
            if trace is not None:
                trace.append({"i0": i0, "j0": j0, "m": run.m.copy(), "l": run.l.copy(), "acc": run.acc.copy()})
        O[rows], L[rows] = finish(run, np.log2 if mistake == "lse_log2" else np.log,
                                  normalised=normalised or mistake == "normalize_in_loop")
    return O, L


def online_softmax_row(scores, values, block: int):
    """One row of scalar scores and scalar values folded block by block.

    Returns (per-block list of (m, factor applied to the running sum, l, output
    so far), final output): the one-row exercise of the lesson page's
    "Practice" section.
    """
    s = np.asarray(scores, dtype=np.float64)[None, :]
    v = np.asarray(values, dtype=np.float64)[:, None]
    run = Partial.empty(1, 1)
    steps = []
    for s0 in range(0, s.shape[1], block):
        blk = block_partial(s[:, s0:s0 + block], v[s0:s0 + block])
        factor = float(np.exp(run.m[0] - _finite_ref(np.maximum(run.m, blk.m))[0]))
        run = merge(run, blk)
        steps.append((float(run.m[0]), factor, float(run.l[0]), float(finish(run)[0][0, 0])))
    return steps, float(finish(run)[0][0, 0])
