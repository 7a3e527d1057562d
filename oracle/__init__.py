"""Plain CPU fp64 oracle for block-sparse attention scoring.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never imports it and shares no code with it.

Every function works on fp64 NumPy arrays holding the exact values of the
inputs (bf16 or fp32 values upcast to fp64), follows the definition written
on the pages step by step, and uses no blocking, fusion or reordering beyond
that definition:

* ``scoring``   - PARK's query-preserving block scorer (PARK: Accurate Block
  Retrieval for Sparse Attention in Video Diffusion Transformers, Abstract).
* ``selection`` - online top-p block selection with per-head thresholds
  (HASTE abstract; HEART abstract).
* ``attention`` - attention restricted to the retrieved blocks, written as
  dense softmax attention under an explicit token mask (PARK, Abstract).
* ``drift``     - the per-head query-key drift signal and the refresh rule of
  Temporal Mask Reuse (HEART abstract; HASTE abstract).
* ``trajectory``- estimate once, cache, reuse, refresh on drift (RAPID
  abstract; HEART abstract), plus RAPID's Turbo re-selection on cached scores.
* ``retrieval`` - block retrieval accuracy: each query block's dense attention
  mass per key block, and the mass a selection captures (PARK, Abstract).
* ``clustering`` - PARK's query-aware key clustering: k-means in the metric
  the current queries induce, clusters as key blocks, their scores and
  attention (PARK, Abstract).
* ``correction`` - the cached correction of sparse attention by the attention
  over its omitted blocks, weighted by the fresh sparse statistics (RECAP
  abstract).

What pins each function (closed forms, invariants, brute force, independent
library routines) is in ``tests/test_oracle.py``; no function here is left
parity-unpinned.
"""
from .blocks import block_bounds, num_blocks
from .scoring import pool_keys, score_blocks, score_blocks_pooled_query, score_head
from .selection import select_row, select_topp, density
from .attention import block_sparse_attention, token_mask
from .drift import drift, refresh_decision
from .trajectory import cache_trajectory, turbo_schedule
from .retrieval import captured_mass, dense_block_mass
from .correction import complement_lists, corrected_trajectory, merge_partial, omitted_attention
from .clustering import (assign, cluster_attention, cluster_keys, cluster_order, cluster_scores, kmeans,
                         metric_distance, query_gram, update)

__all__ = [
    "block_bounds", "num_blocks", "pool_keys", "score_blocks", "score_head",
    "score_blocks_pooled_query", "select_row", "select_topp", "density",
    "block_sparse_attention", "token_mask", "drift", "refresh_decision",
    "cache_trajectory", "turbo_schedule", "dense_block_mass", "captured_mass",
    "complement_lists", "omitted_attention", "merge_partial", "corrected_trajectory",
    "query_gram", "metric_distance", "assign", "update", "kmeans", "cluster_order", "cluster_keys",
    "cluster_scores", "cluster_attention",
]
