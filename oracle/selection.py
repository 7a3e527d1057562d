"""Top-p block selection, fp64 (oracle; test infrastructure only).

HASTE (Training-Free Video Diffusion Acceleration via Head-Wise Adaptive
Sparse Attention), Abstract: masks come from online top-p selection, and each
head may have its own top-p threshold; HEART (Exploiting Head Heterogeneity
in Sparse Attention for Video Diffusion), Abstract, likewise assigns each
head its own threshold under a global sparsity budget.

Readings where the pages are silent:
* a row keeps the smallest prefix of its key blocks, taken in order of
  decreasing score, whose score mass reaches ``p`` (inclusive ``>=``); at
  least one block; ``p >= 1`` keeps every block;
* equal scores are taken in increasing key-block index;
* no block is forced in (no diagonal or sink blocks);
* the global budget lives in the per-head ``p``; the only run-time budget is
  an optional per-row cap ``max_blocks`` (0 means none).

The threshold ``p`` is the float32 value handed to the library, compared in
fp64 with the fp64 running sum.
"""
import numpy as np


def select_row(s: np.ndarray, p: float, max_blocks: int = 0):
    """One row of scores -> (sorted ascending selected indices, k*, order, csum)."""
    nb = s.shape[0]
    j = np.arange(nb)
    order = np.lexsort((j, -s))          # score descending, then index ascending
    csum = np.cumsum(s[order])           # sequential fp64 running mass
    p64 = float(np.float32(p))
    if p64 >= 1.0:
        kstar = nb
    else:
        hit = np.nonzero(csum >= p64)[0]
        kstar = int(hit[0]) + 1 if hit.size else nb
    if max_blocks > 0:
        kstar = min(kstar, max_blocks)
    sel = np.sort(order[:kstar])
    return sel, kstar, order, csum


def select_topp(scores: np.ndarray, top_p, max_blocks: int = 0):
    """``S [H, NB, NB]`` and ``p [H]`` -> (mask u8, counts i32, lists)."""
    h, nbq, nb = scores.shape
    p = np.broadcast_to(np.asarray(top_p, np.float32), (h,))
    mask = np.zeros((h, nbq, nb), np.uint8)
    counts = np.zeros((h, nbq), np.int32)
    lists = []
    for a in range(h):
        rows = []
        for i in range(nbq):
            sel, kstar, _, _ = select_row(scores[a, i], float(p[a]), max_blocks)
            mask[a, i, sel] = 1
            counts[a, i] = kstar
            rows.append(sel.astype(np.int32))
        lists.append(rows)
    return mask, counts, lists


def density(counts: np.ndarray, nb: int) -> np.ndarray:
    """Fraction of (query block, key block) pairs kept, per head."""
    return counts.reshape(counts.shape[0], -1).sum(axis=1) / float(nb * nb)
