"""Cross-step mask reuse: a host loop over the four library calls.

RAPID (Reusing Attention Sparsity with Inter-step Adaptation for Efficient
Video Diffusion), Abstract: estimate block importance once, cache the scores
and the mask, reuse them in later denoising steps; the cached scores also
allow a multi-stage re-pruning (Turbo mode).  HEART (Exploiting Head
Heterogeneity in Sparse Attention for Video Diffusion), Abstract: per head,
refresh the cached mask only when its query-key drift exceeds a threshold.

With ``correction=True`` the cache also keeps RECAP's correction (Reciprocal
Sparse Attention and Hierarchical Caching for Efficient Video Diffusion,
Abstract): whenever a head's mask is refreshed, the attention over the blocks
its lists leave out is computed on that step's inputs and cached; every step
joins the fresh sparse output with the cached part, weighted by their
log-sum-exps.

All state lives in device buffers owned by this object; every step enqueues
the library calls on the current stream and never synchronises.  The refresh
flags stay on the device and gate the scoring and selection kernels (and the
refresh of the cached correction).
"""
from __future__ import annotations

import torch

from . import binding as B


class MaskCache:
    def __init__(self, problem: B.Problem, top_p: torch.Tensor, threshold: float,
                 max_blocks: int = 0, device=None, correction: bool = False):
        p = problem
        dev = device if device is not None else top_p.device
        nb = p.nblocks
        dt = torch.bfloat16 if p.dtype == B.RSA_BF16 else torch.float32
        self.p = p
        self.top_p = top_p
        self.threshold = float(threshold)
        self.max_blocks = int(max_blocks)
        self.scores = torch.zeros((p.heads, nb, nb), dtype=torch.float32, device=dev)
        self.mask = torch.zeros((p.heads, nb, nb), dtype=torch.uint8, device=dev)
        self.counts = torch.zeros((p.heads, nb), dtype=torch.int32, device=dev)
        self.block_idx = torch.zeros((p.heads, nb, nb), dtype=torch.int32, device=dev)
        self.density = torch.zeros((p.heads,), dtype=torch.float32, device=dev)
        self.q_ref = torch.zeros((p.heads, p.tokens, p.head_dim), dtype=dt, device=dev)
        self.k_ref = torch.zeros_like(self.q_ref)
        self.drift = torch.zeros((p.heads,), dtype=torch.float32, device=dev)
        self.refresh = torch.zeros((p.heads,), dtype=torch.uint8, device=dev)
        self.score_ws = torch.empty(max(1, B.workspace_bytes(p, B.OP_SCORE)), dtype=torch.uint8, device=dev)
        self.drift_ws = torch.empty(max(1, B.workspace_bytes(p, B.OP_DRIFT)), dtype=torch.uint8, device=dev)
        self.attn_ws = torch.empty(max(1, B.workspace_bytes(p, B.OP_ATTN)), dtype=torch.uint8, device=dev)
        self.steps = 0
        self.correction = bool(correction)
        self.corr_out = self.corr_lse = None
        self._corr_all = True          # the next refresh recomputes every head's correction
        if self.correction:
            self.corr_out = torch.zeros_like(self.q_ref)
            self.corr_lse = torch.full((p.heads, p.tokens), float("-inf"), dtype=torch.float32, device=dev)

    def update_mask(self, q: torch.Tensor, k: torch.Tensor):
        """Drift check, then re-score / re-select the refreshed heads (all at step 0).

        Returns the head flags the refresh used (None: every head)."""
        B.mask_drift(q, k, self.q_ref, self.k_ref, self.p, self.threshold, update_ref=True,
                     drift=self.drift, refresh=self.refresh, workspace=self.drift_ws)
        active = None if self.steps == 0 else self.refresh
        B.score_blocks(q, k, self.p, head_active=active, out=self.scores, workspace=self.score_ws)
        B.select_topp(self.scores, self.top_p, self.p, self.max_blocks, head_active=active,
                      mask=self.mask, counts=self.counts, block_idx=self.block_idx,
                      density=self.density)
        self.steps += 1
        return active

    def step(self, q, k, v, out=None, lse=None):
        """One denoising step's attention with the cached (or refreshed) mask;
        with the correction on, joined with the cached omitted part."""
        active = self.update_mask(q, k)
        if not self.correction:
            return B.block_sparse_attn(q, k, v, self.counts, self.block_idx, self.p, out=out,
                                       lse=lse, workspace=self.attn_ws)
        B.attn_omitted(q, k, v, self.counts, self.block_idx, self.p,
                       head_active=None if self._corr_all else active, out=self.corr_out,
                       lse=self.corr_lse, workspace=self.attn_ws)
        self._corr_all = False
        # the sparse pass joined with the cached part inside the attention kernel
        return B.block_sparse_attn_corrected(q, k, v, self.counts, self.block_idx, self.corr_out, self.corr_lse,
                                             self.p, out=out, lse=lse, workspace=self.attn_ws)

    def turbo(self, top_p: torch.Tensor, max_blocks: int | None = None):
        """RAPID Turbo mode: re-select every head on the cached scores (no re-scoring)."""
        self.top_p = top_p
        B.select_topp(self.scores, top_p, self.p, self.max_blocks if max_blocks is None else max_blocks,
                      mask=self.mask, counts=self.counts, block_idx=self.block_idx,
                      density=self.density)
        # every list changed: the cached omitted parts no longer match them
        self._corr_all = True
