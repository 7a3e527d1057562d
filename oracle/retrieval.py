"""Block retrieval accuracy, fp64 (oracle; test infrastructure only).

PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
Transformers), Abstract: the point of the method is to retrieve the key blocks
that matter to each query block more accurately than a scorer that averages
the queries before the softmax.  The yardstick used here is the dense
attention itself: how much of each query block's full-softmax attention mass
falls on each key block, and how much of that mass a scorer's selection
keeps.

Readings where the page is silent (the page gives no metric):
* the reference importance of key block J for query block I is the mean, over
  the queries of I, of the dense softmax mass (over all N keys) on the tokens
  of J;
* a selection is judged by the mass it captures, averaged over query blocks;
  scorers are compared at equal density (the same number of blocks per row).
"""
import numpy as np

from .blocks import block_bounds, num_blocks


def dense_block_mass(q: np.ndarray, k: np.ndarray, b: int, scale: float | None = None,
                     query_blocks=None) -> np.ndarray:
    """One head: ``M[I, J]`` for all (or the listed) query blocks.

    ``q, k [N, D]``.  Row I: for every query of block I the softmax of
    ``scale * <q_i, k_t>`` over all N keys, summed over the tokens of each key
    block, then averaged over the queries of I.  Every row sums to 1.
    """
    n, d = q.shape
    s = 1.0 / np.sqrt(d) if scale is None else scale
    nb = num_blocks(n, b)
    starts = np.array([block_bounds(j, n, b)[0] for j in range(nb)])
    rows = range(nb) if query_blocks is None else query_blocks
    out = []
    for i in rows:
        lo, hi = block_bounds(i, n, b)
        logits = s * (q[lo:hi] @ k.T)                     # [b_I, N]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        p = e / e.sum(axis=1, keepdims=True)              # dense softmax of each query
        per_block = np.add.reduceat(p, starts, axis=1)    # [b_I, NB]: mass on each key block
        out.append(per_block.mean(axis=0))
    return np.stack(out)


def captured_mass(mass: np.ndarray, lists) -> float:
    """Mean over rows I of the dense mass held by the blocks ``lists[I]``."""
    return float(np.mean([mass[i, np.asarray(l, dtype=int)].sum() for i, l in enumerate(lists)]))
