"""Cross-step mask caching, fp64 (oracle; test infrastructure only).

RAPID (Reusing Attention Sparsity with Inter-step Adaptation for Efficient
Video Diffusion), Abstract: estimate block importance once, early, and cache
the scores and the mask for reuse in later steps; the cached scores also
allow a multi-stage pruning (Turbo mode) as the needed density decays.
HEART, Abstract: per head, keep the cached mask while its query-key drift
stays at or below a threshold and refresh it when the drift exceeds it.

Reading: at step 0 every head is scored and selected and its (Q, K) is
snapshotted; at step s >= 1 the drift is measured against each head's
snapshot, refreshed heads are re-scored and re-selected on the current
(Q, K) and re-snapshotted, other heads keep their cached scores and lists;
attention always runs on the current (Q, K, V) with the list in force.
"""
import numpy as np

from .scoring import score_head
from .selection import select_row
from .drift import drift, refresh_decision


def _select_head(s_head, p, max_blocks):
    rows = [select_row(s_head[i], p, max_blocks) for i in range(s_head.shape[0])]
    return [r[0].astype(np.int32) for r in rows], np.array([r[1] for r in rows], np.int32)


def cache_trajectory(steps, b: int, top_p, tau: float, scale: float | None = None,
                     max_blocks: int = 0):
    """Run the reuse policy over ``steps`` = iterable of (q, k) fp64 ``[H, N, D]``.

    Yields per step: ``(refresh [H] u8, drift [H] or None, lists, counts, scores)``
    where ``lists[h][I]`` is the block list in force for attention at that step.
    """
    q_ref = k_ref = None
    cache_s = cache_l = cache_c = None
    for s, (q, k) in enumerate(steps):
        h, n, d = q.shape
        sc = 1.0 / np.sqrt(d) if scale is None else scale
        p = np.broadcast_to(np.asarray(top_p, np.float32), (h,))
        if s == 0:
            dvals = None
            refresh = np.ones(h, np.uint8)
            cache_s = [None] * h
            cache_l = [None] * h
            cache_c = [None] * h
            q_ref = q.copy()
            k_ref = k.copy()
        else:
            dvals = drift(q, k, q_ref, k_ref)
            refresh = refresh_decision(dvals, tau)
        for a in range(h):
            if refresh[a]:
                cache_s[a] = score_head(q[a], k[a], b, sc)
                cache_l[a], cache_c[a] = _select_head(cache_s[a], float(p[a]), max_blocks)
                q_ref[a] = q[a]
                k_ref[a] = k[a]
        yield refresh, dvals, [list(x) for x in cache_l], np.stack(cache_c), np.stack(cache_s)


def turbo_schedule(scores: np.ndarray, p_stages, max_blocks: int = 0):
    """RAPID Turbo mode: re-select on cached scores for a decaying ``p`` schedule.

    Returns the per-stage (mask, counts) for ``p_stages`` (each entry [H] or a
    scalar); no re-scoring happens.
    """
    from .selection import select_topp
    out = []
    for p in p_stages:
        mask, counts, _ = select_topp(scores, p, max_blocks)
        out.append((mask, counts))
    return out
