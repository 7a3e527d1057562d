"""PARK block scorer, fp64 (oracle; test infrastructure only).

PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
Transformers), Abstract: retrieval starts from the averaged representation of
each key block; PARK keeps every original query, normalises each query's
attention over the key blocks on its own, and then averages those
distributions inside each query block.  The Summary restates this as keeping
the unique information of each query.

Readings where the page is silent:
* logit scale: the same ``softmax_scale`` as attention (default 1/sqrt(D));
* the mean of a ragged last block is over the tokens it actually holds, and
  no block-size weight enters the block softmax.
"""
import numpy as np

from .blocks import block_bounds, num_blocks


def pool_keys(k: np.ndarray, b: int) -> np.ndarray:
    """Mean of the keys in each key block: ``[N, D] -> [NB, D]``."""
    n, d = k.shape
    nb = num_blocks(n, b)
    out = np.empty((nb, d), np.float64)
    for j in range(nb):
        lo, hi = block_bounds(j, n, b)
        out[j] = k[lo:hi].sum(axis=0) / (hi - lo)
    return out


def _row_softmax(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=1, keepdims=True)


def score_head(q: np.ndarray, k: np.ndarray, b: int, scale: float,
               query_blocks=None) -> np.ndarray:
    """Scores of one head, ``S[I, J]``, for all (or the listed) query blocks.

    1. pool the key blocks (``pool_keys``);
    2. logits of every query against every pooled key block, times ``scale``;
    3. softmax of each query's logits over the key blocks;
    4. mean of those distributions over the queries of each query block.
    """
    n, _ = q.shape
    nb = num_blocks(n, b)
    kbar = pool_keys(k, b)
    rows = range(nb) if query_blocks is None else query_blocks
    out = np.empty((len(rows), nb), np.float64)
    for r, i in enumerate(rows):
        lo, hi = block_bounds(i, n, b)
        logits = scale * (q[lo:hi] @ kbar.T)         # [b_I, NB]
        p = _row_softmax(logits)                      # each query on its own
        out[r] = p.mean(axis=0)                       # average within block I
    return out


def score_blocks(q: np.ndarray, k: np.ndarray, b: int, scale: float | None = None) -> np.ndarray:
    """All heads: ``q, k [H, N, D] -> S [H, NB, NB]``."""
    h, n, d = q.shape
    s = 1.0 / np.sqrt(d) if scale is None else scale
    return np.stack([score_head(q[i], k[i], b, s) for i in range(h)])


def score_blocks_pooled_query(q: np.ndarray, k: np.ndarray, b: int,
                              scale: float | None = None) -> np.ndarray:
    """The scorer PARK argues against (query-side aggregation mismatch).

    PARK, Abstract: averaging the queries of a block *before* the softmax
    loses their individual preferences.  This comparison scorer pools both
    sides and takes one softmax per query block.  It is used only to measure
    retrieval accuracy against PARK's scorer.
    """
    h, n, d = q.shape
    s = 1.0 / np.sqrt(d) if scale is None else scale
    out = []
    for i in range(h):
        qbar = pool_keys(q[i], b)        # same block mean, applied to queries
        kbar = pool_keys(k[i], b)
        out.append(_row_softmax(s * (qbar @ kbar.T)))
    return np.stack(out)
