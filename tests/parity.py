"""Comparison helpers for GPU-vs-oracle parity (test infrastructure).

Top-p selection has several correct answers only at ties.  A row (h, I) is a
tie row when, under the oracle's fp64 scores S and k* = the oracle's count:
  |C_{k*} - p| <= TIE, or k* > 1 and |C_{k*-1} - p| <= TIE, or
  k* < NB and |S_(k*) - S_(k*+1)| <= TIE  (sorted descending; 1-based),
with C the running mass in sorted order and TIE = 1e-6.  On a tie row the
GPU's set is accepted when it is still a valid top-p set under the oracle's
scores: mass >= p - TIE and size in {k*-1, k*, k*+1}.  Every such row is
reported.  Any other difference is a failure.
"""
from __future__ import annotations

import numpy as np

import oracle as O

TIE = 1e-6


def classify_row(s_row: np.ndarray, p: float, gpu_sel, max_blocks: int = 0):
    """-> ("equal" | "tie" | "fail", oracle_selection)."""
    sel, kstar, order, csum = O.select_row(s_row, p, max_blocks)
    g = np.asarray(sorted(int(x) for x in gpu_sel))
    if g.shape == sel.shape and (g == sel).all():
        return "equal", sel
    nb = s_row.shape[0]
    p64 = float(np.float32(p))
    srt = s_row[order]
    capped = max_blocks > 0 and kstar == max_blocks and (csum[kstar - 1] < p64 or kstar < nb)
    tie = False
    if not capped:
        tie |= abs(csum[kstar - 1] - p64) <= TIE
        tie |= kstar > 1 and abs(csum[kstar - 2] - p64) <= TIE
    tie |= kstar < nb and abs(srt[kstar - 1] - srt[kstar]) <= TIE
    if tie and g.size:
        mass = float(s_row[g].sum())
        ok_mass = capped or p64 >= 1.0 or mass >= p64 - TIE
        if ok_mass and abs(g.size - kstar) <= 1 and len(set(g.tolist())) == g.size:
            return "tie", sel
    return "fail", sel


def check_rows(s_oracle, p_heads, gpu_lists, rows, max_blocks=0):
    """Classify rows [(h, I)]; returns counts and the list of tie/fail rows."""
    out = {"equal": 0, "tie": 0, "fail": 0}
    ties, fails = [], []
    for (h, i), srow, glist in zip(rows, s_oracle, gpu_lists):
        kind, sel = classify_row(srow, float(p_heads[h]), glist, max_blocks)
        out[kind] += 1
        if kind == "tie":
            ties.append((h, i))
        elif kind == "fail":
            fails.append((h, i, list(map(int, glist)), list(map(int, sel))))
    return out, ties, fails


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def gpu_lists_from(counts_row: np.ndarray, idx_rows: np.ndarray):
    """Per-row block lists from the library's compacted output."""
    return [idx_rows[r, :counts_row[r]] for r in range(counts_row.shape[0])]
