"""RAPID Turbo mode on the GPU: re-selection on cached scores, no re-scoring.

RAPID (Reusing Attention Sparsity with Inter-step Adaptation for Efficient
Video Diffusion), Abstract: the cached scores allow a multi-stage pruning as
the needed density decays.  Each stage runs rsa_select_topp on the cache's
scores with a lower threshold; on those identical fp32 scores the masks must
equal the oracle's bit for bit, stages must be nested and the density must
not grow.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import block_sparse_attention_scoring_amd as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("name", ["wan13b_480p", "wan14b_720p"])
def test_turbo_reselection_matches_oracle(name):
    wl = W.CONFIGS[name].scaled(heads=4, name=f"{name}-4h")
    print(f"[gpu] turbo {wl.name}", flush=True)
    inp = W.make_inputs(wl)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    p = R.make_problem(q, wl.grid, wl.block)
    cache = R.MaskCache(p, torch.from_numpy(inp.top_p).to(DEV), threshold=0.05)
    cache.step(q, k, v)
    scores = cache.scores.cpu().numpy().astype(np.float64)
    stages = [np.float32(x) * inp.top_p for x in (1.0, 0.95, 0.85, 0.7)]
    prev_mask, prev_dens = None, None
    for ps in stages:
        cache.turbo(torch.from_numpy(ps.astype(np.float32)).to(DEV))
        torch.cuda.synchronize()
        mask = cache.mask.cpu().numpy()
        dens = cache.density.cpu().numpy()
        m_or, c_or, _ = O.select_topp(scores, ps.astype(np.float32))
        assert (mask == m_or).all() and (cache.counts.cpu().numpy() == c_or).all()
        if prev_mask is not None:
            assert (mask <= prev_mask).all()
            assert (dens <= prev_dens + 1e-7).all()
        prev_mask, prev_dens = mask, dens
        out, _ = R.block_sparse_attn(q, k, v, cache.counts, cache.block_idx, p)
        assert torch.isfinite(out.float()).all()
    print(f"[gpu] turbo {wl.name}: final density {prev_dens.round(3).tolist()}", flush=True)
