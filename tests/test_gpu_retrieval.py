"""GPU parity of the retrieval-accuracy calls against the fp64 oracle.

rsa_dense_block_mass: |dM| <= 1e-5 and every row sums to 1 within 1e-5.  The
bound: logits are exact products of the inputs accumulated in fp32; the row
normaliser is an fp64 sum of fp32 partial sums and the resulting log2-sum
is rounded to fp32 (|lse2| <= ~40, one ulp ~4e-6, so each probability is off
by <= ~3e-6 relative); block sums of fp32 probabilities add ~1e-6 relative.
rsa_score_blocks_pooled: |dS| <= 1e-6 (block means rounded once to fp32,
fp64 logits and softmax).
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
MASS_TOL = 1e-5
POOLED_TOL = 1e-6

CASES = {
    # name: (heads, grid, head_dim, block, dtype)
    "bf16_d128_b64": (2, (6, 20, 83), 128, 64, "bf16"),    # N=9960, NB=156, last block 40
    "bf16_d128_b128": (2, (6, 20, 83), 128, 128, "bf16"),  # NB=78, last block 104
    "bf16_d64_b128": (2, (5, 16, 51), 64, 128, "bf16"),    # NB=32, last block 112
    "bf16_d64_b64": (3, (4, 9, 37), 64, 64, "bf16"),       # NB=21, last block 52
    "bf16_d128_b128_short": (3, (2, 13, 31), 128, 128, "bf16"),  # NB=7, last block 38
    "fp32_d128_b128": (2, (3, 10, 29), 128, 128, "fp32"),  # NB=7, last block 102
    "fp32_d64_b64": (1, (4, 8, 8), 64, 64, "fp32"),        # the tiny shape
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def workload(name):
    h, grid, d, b, dt = CASES[name]
    return W.Workload(200 + sorted(CASES).index(name), name, h, grid, d, b, dt, (0.8, 0.9, 0.95))


@pytest.mark.parametrize("name", sorted(CASES))
def test_dense_block_mass_and_pooled_scores_match_oracle(name):
    wl = workload(name)
    inp = W.make_inputs(wl)
    say(f"[gpu] retrieval {name}: heads={wl.heads} tokens={wl.tokens} D={wl.head_dim} B={wl.block} NB={wl.nblocks}")
    q, k = inp.q.to(DEV), inp.k.to(DEV)
    p = R.make_problem(q, wl.grid, wl.block)
    mass = R.dense_block_mass(q, k, p)
    pooled = R.score_blocks_pooled(q, k, p)
    torch.cuda.synchronize()
    m_h, s_h = mass.cpu().numpy().astype(np.float64), pooled.cpu().numpy().astype(np.float64)
    q64, k64 = W.to_f64(inp.q), W.to_f64(inp.k)
    m_or = np.stack([O.dense_block_mass(q64[h], k64[h], wl.block) for h in range(wl.heads)])
    s_or = O.score_blocks_pooled_query(q64, k64, wl.block)
    dm, ds = np.abs(m_h - m_or).max(), np.abs(s_h - s_or).max()
    rows = np.abs(m_h.sum(-1) - 1).max()
    say(f"[gpu] {name}: max|dM| {dm:.2e} (row sums off by {rows:.2e}), max|dS_pooled| {ds:.2e}")
    assert dm <= MASS_TOL and rows <= MASS_TOL
    assert ds <= POOLED_TOL


def test_full_size_720p_sampled_rows():
    """720p shape: every row of the dense mass sums to 1; sampled query
    blocks of two heads against the oracle; pooled scores of two heads."""
    wl = W.CONFIGS["wan14b_720p"]
    inp = W.make_inputs(wl, heads=[0, 27])
    say(f"[gpu] retrieval full size: heads {inp.q.shape[0]} tokens={wl.tokens} NB={wl.nblocks}")
    q, k = inp.q.to(DEV), inp.k.to(DEV)
    p = R.make_problem(q, wl.grid, wl.block)
    mass = R.dense_block_mass(q, k, p)
    pooled = R.score_blocks_pooled(q, k, p)
    torch.cuda.synchronize()
    m_h, s_h = mass.cpu().numpy().astype(np.float64), pooled.cpu().numpy().astype(np.float64)
    assert np.abs(m_h.sum(-1) - 1).max() <= MASS_TOL
    q64, k64 = W.to_f64(inp.q), W.to_f64(inp.k)
    nb = wl.nblocks
    worst = 0.0
    for h in range(2):
        rows = [0, nb // 2, nb - 1]
        m_or = O.dense_block_mass(q64[h], k64[h], wl.block, query_blocks=rows)
        worst = max(worst, float(np.abs(m_h[h, rows] - m_or).max()))
    ds = float(np.abs(s_h - O.score_blocks_pooled_query(q64, k64, wl.block)).max())
    say(f"[gpu] 720p: sampled max|dM| {worst:.2e}, pooled max|dS| {ds:.2e}")
    assert worst <= MASS_TOL and ds <= POOLED_TOL
