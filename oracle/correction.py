"""Cached correction of sparse attention by its omitted key blocks, fp64
(oracle; test infrastructure only).

RECAP (Reciprocal Sparse Attention and Hierarchical Caching for Efficient Video
Diffusion), Abstract: sparse attention leaves interactions out; a dense
refinement, computed now and then and cached, corrects those omitted
interactions in later sparse estimates, while the statistics of each fresh
sparse pass follow the changing inputs and govern how much the ageing
correction counts.

The abstract gives no formula.  Reading used here:

* The omitted interactions of query block ``I`` are the key blocks its list
  leaves out (the complement list).  The refinement computed at a refresh is
  the attention of every query over those keys alone: an output ``O_o`` and
  its log-sum-exp ``lse_o``.  It is cached per head and recomputed whenever
  that head's mask is refreshed, so it always covers exactly the complement of
  the list in force.
* The fresh sparse statistics are the sparse pass's own output ``O_s`` and
  log-sum-exp ``lse_s``.
* The corrected output joins the two as a softmax over the union of two
  disjoint key sets does: weights ``exp(lse_s)`` and ``exp(lse_o)``, normalised
  to one.  On the inputs of the refresh itself this is dense attention
  exactly; later, a growing or shrinking ``lse_s`` lowers or raises the weight
  of the cached part.
"""
import numpy as np

from .attention import block_sparse_attention
from .blocks import num_blocks
from .trajectory import cache_trajectory


def complement_lists(lists, nb: int):
    """Per row, the key blocks in ``[0, nb)`` that the row's list leaves out,
    ascending.  A list is read as a set: order and repeats do not matter and
    entries outside ``[0, nb)`` are ignored."""
    out = []
    for row in lists:
        keep = np.ones(nb, bool)
        for j in row:
            j = int(j)
            if 0 <= j < nb:
                keep[j] = False
        out.append(np.flatnonzero(keep).astype(np.int32))
    return out


def omitted_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, b: int, lists,
                      scale: float | None = None):
    """One head: attention of every query over the key blocks its list omits.

    Returns ``(out [N, D], lse [N])``; a row whose list covers every block has
    nothing omitted and gets a zero output and ``lse = -inf``.
    """
    n = q.shape[0]
    return block_sparse_attention(q, k, v, b, complement_lists(lists, num_blocks(n, b)), scale)


def merge_partial(o_a: np.ndarray, lse_a: np.ndarray, o_b: np.ndarray, lse_b: np.ndarray):
    """Attention over the union of two disjoint key sets from the attention over
    each: ``(out [rows, D], lse [rows])``.

    Each part's softmax is normalised over its own keys; ``exp(lse)`` is the
    part's total of exponentiated logits, so the union's softmax gives part
    ``a`` the weight ``exp(lse_a) / (exp(lse_a) + exp(lse_b))``.  A part with
    ``lse = -inf`` (no keys) has weight zero; two such parts give a zero row
    and ``lse = -inf``.
    """
    lse = np.logaddexp(lse_a, lse_b)
    out = np.zeros(np.broadcast_shapes(o_a.shape, o_b.shape))
    live = np.isfinite(lse)
    wa = np.exp(lse_a[live] - lse[live])[:, None]
    wb = np.exp(lse_b[live] - lse[live])[:, None]
    out[live] = wa * o_a[live] + wb * o_b[live]
    return out, lse


def corrected_trajectory(steps, b: int, top_p, tau: float, scale: float | None = None,
                         max_blocks: int = 0):
    """Mask caching with the cached correction, over ``steps`` = sequence of
    ``(q, k, v)`` fp64 ``[H, N, D]``.

    The masks follow ``cache_trajectory`` (drift-gated per-head refresh).  When
    head ``h`` is refreshed, the attention over its omitted blocks is computed
    on that step's ``(q, k, v)`` and cached.  Every step, the fresh sparse
    attention over the list in force is merged with the cached omitted part.

    Yields per step ``(refresh [H] u8, lists, out [H,N,D], lse [H,N],
    sparse_out [H,N,D], sparse_lse [H,N])``.
    """
    steps = list(steps)
    masks = cache_trajectory([(q, k) for q, k, _ in steps], b, top_p, tau, scale, max_blocks)
    cached = None
    for (q, k, v), (refresh, _, lists, _, _) in zip(steps, masks):
        h = q.shape[0]
        if cached is None:
            cached = [None] * h
        outs, lses, souts, slses = [], [], [], []
        for a in range(h):
            if refresh[a]:
                cached[a] = omitted_attention(q[a], k[a], v[a], b, lists[a], scale)
            o_s, l_s = block_sparse_attention(q[a], k[a], v[a], b, lists[a], scale)
            o, l = merge_partial(o_s, l_s, *cached[a])
            outs.append(o)
            lses.append(l)
            souts.append(o_s)
            slses.append(l_s)
        yield refresh, lists, np.stack(outs), np.stack(lses), np.stack(souts), np.stack(slses)
