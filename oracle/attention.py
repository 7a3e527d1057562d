"""Attention restricted to retrieved blocks, fp64 (oracle; test infrastructure only).

PARK, Abstract: sparse attention retrieves the important blocks and computes
attention only inside them.  Written here as dense softmax attention under an
explicit token mask: query ``i`` of block ``I`` may see exactly the tokens of
the key blocks listed for ``(h, I)``; the softmax is normalised over those
tokens only.  HEART's abstract notes that the sparse kernel itself is not
changed by mask reuse, so attention depends only on the block list it is given.

Reading for an empty list: the output row is zero and its log-sum-exp is -inf.
"""
import numpy as np

from .blocks import block_bounds, num_blocks


def token_mask(n: int, b: int, blocks) -> np.ndarray:
    """Boolean mask over the ``n`` key tokens covered by the listed key blocks."""
    m = np.zeros(n, bool)
    for j in blocks:
        lo, hi = block_bounds(int(j), n, b)
        m[lo:hi] = True
    return m


def block_sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int,
                           lists, scale: float | None = None, query_blocks=None):
    """One head.  ``q,k,v [N, D]``; ``lists[I]`` = selected key blocks of row I.

    Returns ``(out [rows, D], lse [rows])`` for the listed query blocks (all by
    default), stacked in that order.
    """
    n, d = q.shape
    s = 1.0 / np.sqrt(d) if scale is None else scale
    nb = num_blocks(n, b)
    rows = range(nb) if query_blocks is None else query_blocks
    outs, lses = [], []
    for i in rows:
        lo, hi = block_bounds(i, n, b)
        allowed = np.flatnonzero(token_mask(n, b, lists[i]))
        if allowed.size == 0:
            outs.append(np.zeros((hi - lo, d)))
            lses.append(np.full(hi - lo, -np.inf))
            continue
        logits = s * (q[lo:hi] @ k[allowed].T)
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        z = e.sum(axis=1, keepdims=True)
        outs.append((e / z) @ v[allowed])
        lses.append((m + np.log(z))[:, 0])
    return np.concatenate(outs), np.concatenate(lses)
