"""Query-aware key clustering, fp64 (oracle; test infrastructure only).

PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
Transformers), Abstract: clustering keys by Euclidean distance in their own
space can put keys that the current queries score differently into one
cluster, whose mean then misrepresents them; PARK transforms the keys with
information from the current queries before clustering, so that keys with
similar query-key scores end up together, and uses the clusters' mean
representations for block retrieval.

The abstract gives neither the transform nor the clustering algorithm.
Reading used here:

* The metric is the one the current queries induce.  With ``G = Q^T Q / N``
  (the mean outer product of the head's N current queries), the squared
  distance of key ``k`` to a point ``c`` is ``(k - c)^T G (k - c)``, which is
  the mean over the current queries of the squared difference of their scores
  ``<q_i, k> - <q_i, c>``.  Clustering in this metric is Euclidean clustering
  of the transformed keys ``R k`` for any ``R`` with ``R^T R = G``.
* The clustering is Lloyd's k-means: ``NB`` clusters (as many as contiguous
  blocks), started from the means of the contiguous blocks; one iteration
  assigns every key to its nearest centroid in the metric (ties: lowest
  cluster index) and moves every non-empty cluster's centroid to the mean of
  its keys (the mean minimises the metric's squared distances for any G);
  an empty cluster keeps its centroid.
* The clusters are the key blocks.  Query blocks stay the contiguous runs of
  B tokens (PARK keeps every query).  A cluster's representation is its
  centroid; PARK's score of cluster J for query block I is the mean over the
  block's queries of their softmax over the non-empty clusters of
  ``scale * <q_i, c_J>``; an empty cluster scores 0.
* Attention for query block I runs over the keys of the clusters its list
  selects, in the original token order (the order does not change a softmax).
"""
import numpy as np

from .blocks import block_bounds, num_blocks
from .scoring import _row_softmax, pool_keys


def query_gram(q: np.ndarray) -> np.ndarray:
    """``G = Q^T Q / N`` for one head's queries ``[N, D]``."""
    return q.T @ q / q.shape[0]


def metric_distance(x: np.ndarray, c: np.ndarray, g: np.ndarray) -> np.ndarray:
    """``(x - c)^T G (x - c)`` for every row of ``x`` ``[n, D]`` and one point ``c``."""
    d = x - c[None, :]
    return ((d @ g) * d).sum(axis=1)


def assign(k: np.ndarray, centroids: np.ndarray, g: np.ndarray):
    """Nearest centroid of every key in the metric; ties go to the lowest index.

    Returns ``(labels [N] int32, dist [N, C])``."""
    dist = np.stack([metric_distance(k, c, g) for c in centroids], axis=1)
    return np.argmin(dist, axis=1).astype(np.int32), dist


def update(k: np.ndarray, labels: np.ndarray, centroids: np.ndarray):
    """Means of the clusters' keys; an empty cluster keeps its centroid.

    Returns ``(centroids [C, D], sizes [C] int32)``."""
    out = centroids.copy()
    sizes = np.zeros(centroids.shape[0], np.int32)
    for j in range(centroids.shape[0]):
        members = labels == j
        sizes[j] = int(members.sum())
        if sizes[j]:
            out[j] = k[members].mean(axis=0)
    return out, sizes


def kmeans(k: np.ndarray, g: np.ndarray, b: int, iters: int, centroids: np.ndarray | None = None):
    """``iters`` Lloyd iterations in the metric of ``g`` from the contiguous
    block means (or from ``centroids``).

    Returns ``(labels [N], centroids [NB, D], sizes [NB])`` of the last
    iteration: the labels of its assignment and the means of those clusters."""
    c = pool_keys(k, b) if centroids is None else np.asarray(centroids, np.float64).copy()
    labels = sizes = None
    for _ in range(iters):
        labels, _ = assign(k, c, g)
        c, sizes = update(k, labels, c)
    return labels, c, sizes


def cluster_order(labels: np.ndarray) -> np.ndarray:
    """Tokens sorted by (cluster, token index): the keys of each cluster as one
    run, in token order inside the run."""
    return np.argsort(labels, kind="stable").astype(np.int32)


def cluster_keys(q: np.ndarray, k: np.ndarray, b: int, iters: int):
    """The whole clustering of one head: Gram matrix of the current queries,
    then k-means from the contiguous block means.

    Returns ``(labels, centroids, sizes, order)``."""
    labels, c, sizes = kmeans(k, query_gram(q), b, iters)
    return labels, c, sizes, cluster_order(labels)


def cluster_scores(q: np.ndarray, centroids: np.ndarray, sizes: np.ndarray, b: int,
                   scale: float | None = None, query_blocks=None) -> np.ndarray:
    """PARK scores of the clusters for each query block ``[rows, NB]``: per
    query a softmax over the non-empty clusters of ``scale * <q_i, c_J>``, then
    the mean over the block's queries; empty clusters score 0."""
    n, d = q.shape
    s = 1.0 / np.sqrt(d) if scale is None else scale
    live = np.asarray(sizes) > 0
    nb = num_blocks(n, b)
    rows = range(nb) if query_blocks is None else query_blocks
    out = np.zeros((len(rows), centroids.shape[0]))
    for r, i in enumerate(rows):
        lo, hi = block_bounds(i, n, b)
        p = _row_softmax(s * (q[lo:hi] @ centroids[live].T))
        out[r, live] = p.mean(axis=0)
    return out


def cluster_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int, labels: np.ndarray,
                      lists, scale: float | None = None, query_blocks=None):
    """Attention of each query block over the keys of the clusters its list
    selects (a list is a set; entries outside the clusters are ignored).

    Returns ``(out [rows, D], lse [rows])``; an empty selection gives a zero
    row and ``lse = -inf``."""
    n, d = q.shape
    s = 1.0 / np.sqrt(d) if scale is None else scale
    nb = num_blocks(n, b)
    rows = range(nb) if query_blocks is None else query_blocks
    outs, lses = [], []
    for i in rows:
        lo, hi = block_bounds(i, n, b)
        allowed = np.flatnonzero(np.isin(labels, np.asarray(list(lists[i]), np.int64)))
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
