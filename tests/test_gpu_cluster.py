"""PARK's query-aware key clustering on the GPU against the oracle.

PARK (Accurate Block Retrieval for Sparse Attention in Video Diffusion
Transformers), Abstract: keys are clustered in a metric built from the
current queries, and the clusters serve as key blocks.

* rsa_query_gram against the oracle's Gram matrix;
* one Lloyd iteration at a time (rsa_kmeans with iters=1), the oracle given
  the GPU's own starting centroids and Gram matrix: labels equal the oracle's
  nearest centroids except where two centroids are within the assignment's
  stated tolerance (reported); sizes and order are exact for the GPU's labels;
  centroids equal the oracle's means of the GPU's clusters to one fp32
  rounding;
* several iterations in one call equal the same iterations one call at a
  time, bit for bit, and repeat bit for bit;
* keys that are all equal: every key ties, all go to cluster 0.
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

CASES = {
    # name: (heads, grid, head_dim, block, dtype)
    "bf16_d128_b128": (2, (6, 20, 83), 128, 128, "bf16"),  # N=9960: 5 Gram chunks, NB=78 (3 centroid chunks)
    "two_chunks_bf16_d128_b128": (1, (5, 16, 80), 128, 128, "bf16"),  # N=6400, NB=50: an even number (2) of centroid chunks
    "bf16_d128_b64": (2, (3, 10, 41), 128, 64, "bf16"),    # N=1230, NB=20, last block 14
    "bf16_d64_b64": (3, (4, 9, 37), 64, 64, "bf16"),       # N=1332, NB=21
    "fp32_d64_b64": (1, (4, 8, 8), 64, 64, "fp32"),        # the tiny shape
}
# assignment: the GPU forms 2 k.G c_j from fp16 keys (exact) and a 22-bit
# split of 2 G c_j with fp32 sums, like the scorer's logits; a choice that
# differs from the oracle's must be within this share of k^T G k + c^T G c
ASSIGN_TOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().cpu().numpy()


def workload(name):
    h, grid, d, b, dt = CASES[name]
    return W.Workload(300 + sorted(CASES).index(name), name, h, grid, d, b, dt, (0.9,))


class Case:
    def __init__(self, name):
        wl = workload(name)
        self.wl = wl
        inp = W.make_inputs(wl)
        say(f"[gpu] cluster case {name}: heads={wl.heads} tokens={wl.tokens} D={wl.head_dim} "
            f"B={wl.block} NB={wl.nblocks} dtype={wl.dtype}")
        self.q64, self.k64 = W.to_f64(inp.q), W.to_f64(inp.k)
        self.q, self.k = inp.q.to(DEV).contiguous(), inp.k.to(DEV).contiguous()
        self.p = R.make_problem(self.q, wl.grid, wl.block)
        self.gram = R.query_gram(self.q, self.p)
        torch.cuda.synchronize()


_cases = {}


def case(name):
    if name not in _cases:
        _cases[name] = Case(name)
    return _cases[name]


@pytest.mark.parametrize("name", sorted(CASES))
def test_gram_matches_oracle(name):
    c = case(name)
    g = host(c.gram).astype(np.float64)
    for h in range(c.wl.heads):
        want = O.query_gram(c.q64[h])
        err = np.abs(g[h] - want).max() / np.abs(want).max()
        say(f"[gpu] gram {name} h={h}: max rel err {err:.2e}")
        assert err <= 1e-5 if c.wl.dtype == "bf16" else err <= 1e-7


@pytest.mark.parametrize("name", sorted(CASES))
def test_kmeans_iterations_match_oracle(name):
    c = case(name)
    wl, p = c.wl, c.p
    g = host(c.gram).astype(np.float64)
    cent = None
    near_ties = 0
    for it in range(3):
        prev = None if cent is None else cent.clone()
        cent, labels, sizes, order = R.kmeans(c.k, c.gram, p, iters=1, init=it == 0,
                                              centroids=None if it == 0 else prev.clone())
        torch.cuda.synchronize()
        lab, sz, od, cg = host(labels), host(sizes), host(order), host(cent).astype(np.float64)
        for h in range(wl.heads):
            start = O.pool_keys(c.k64[h], wl.block).astype(np.float32).astype(np.float64) if prev is None \
                else host(prev[h]).astype(np.float64)
            want, dist = O.assign(c.k64[h], start, g[h])
            diff = np.flatnonzero(lab[h] != want)
            if diff.size:
                kgk = ((c.k64[h][diff] @ g[h]) * c.k64[h][diff]).sum(1)
                cgc = ((start[lab[h][diff]] @ g[h]) * start[lab[h][diff]]).sum(1)
                gap = dist[diff, lab[h][diff]] - dist[diff, want[diff]]
                assert (gap <= ASSIGN_TOL * (kgk + cgc)).all(), (it, h, diff[:5], gap[:5])
                near_ties += diff.size
            assert (sz[h] == np.bincount(lab[h], minlength=wl.nblocks)).all()
            assert (od[h] == O.cluster_order(lab[h])).all()
            c_or, _ = O.update(c.k64[h], lab[h], start)
            np.testing.assert_allclose(cg[h], c_or, rtol=2 ** -23, atol=1e-30)
        say(f"[gpu] kmeans {name} iteration {it}: non-empty clusters "
            f"{[(int((sz[h] > 0).sum())) for h in range(wl.heads)]}, near-tie labels so far {near_ties}")
    assert near_ties <= max(1, wl.tokens * wl.heads // 1000)


def test_kmeans_several_iterations_in_one_call():
    c = case("bf16_d64_b64")
    out4 = R.kmeans(c.k, c.gram, c.p, iters=4)
    again = R.kmeans(c.k, c.gram, c.p, iters=4)
    cent = R.kmeans(c.k, c.gram, c.p, iters=1)[0]
    for _ in range(3):
        step = R.kmeans(c.k, c.gram, c.p, iters=1, init=False, centroids=cent)
        cent = step[0]
    torch.cuda.synchronize()
    for a, b_, s in zip(out4, again, step):
        assert torch.equal(a, b_) and torch.equal(a, s)


def test_kmeans_all_keys_equal():
    """Every key the same: all block means equal, every key ties with every
    cluster and goes to cluster 0; the other clusters stay empty."""
    wl = W.Workload(330, "equal_keys", 2, (2, 8, 25), 128, 64, "bf16", (0.9,))   # N=400, NB=7
    inp = W.make_inputs(wl)
    q = inp.q.to(DEV)
    k = inp.k[:, :1, :].expand(-1, wl.tokens, -1).contiguous().to(DEV)
    p = R.make_problem(q, wl.grid, wl.block)
    gram = R.query_gram(q, p)
    cent, labels, sizes, order = R.kmeans(k, gram, p, iters=2)
    torch.cuda.synchronize()
    assert (labels == 0).all()
    assert host(sizes).tolist() == [[wl.tokens] + [0] * (wl.nblocks - 1)] * wl.heads
    assert (host(order) == np.arange(wl.tokens)[None, :]).all()
    want = inp.k[:, 0, :].float()
    assert torch.equal(cent.cpu(), want[:, None, :].expand(-1, wl.nblocks, -1))


# (rel L2, max abs) on outputs, max abs on lse: as for block-sparse attention
ATTN_TOL = {"bf16": (1e-2, 3e-2, 1e-3), "fp32": (1e-4, 1e-4, 1e-4)}


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def clustered(c, iters=3):
    if not hasattr(c, "cl"):
        c.cl = R.kmeans(c.k, c.gram, c.p, iters=iters)
        c.v = W.make_inputs(c.wl).v.to(DEV).contiguous()
        c.v64 = W.to_f64(c.v.cpu())
        torch.cuda.synchronize()
    return c.cl


@pytest.mark.parametrize("name", sorted(CASES))
def test_cluster_scores_match_oracle(name):
    c = case(name)
    wl = c.wl
    cent, labels, sizes, order = clustered(c)
    sz = sizes.clone()
    sz[:, 3] = 0                                   # one cluster taken as empty
    for s_in in (sizes, sz):
        S = host(R.score_clusters(c.q, cent, s_in, c.p)).astype(np.float64)
        cg, si = host(cent).astype(np.float64), host(s_in)
        for h in range(wl.heads):
            want = O.cluster_scores(c.q64[h], cg[h], si[h], wl.block)
            err = np.abs(S[h] - want).max()
            say(f"[gpu] cluster scores {name} h={h} empty={int((si[h] == 0).sum())}: max |dS| {err:.2e}")
            assert err <= 1e-6
            assert (S[h][:, si[h] == 0] == 0).all()
            np.testing.assert_allclose(S[h].sum(axis=1), 1.0, atol=1e-5)


def _set_lists(heads, nb, sizes, seed):
    """Cluster lists as sets: shuffled, repeats, out-of-range entries; row 0
    empty, the last row every cluster with an over-long count."""
    rng = np.random.default_rng(seed)
    counts = np.zeros((heads, nb), np.int32)
    idx = np.full((heads, nb, nb), -1, np.int32)
    lists = []
    for h in range(heads):
        rows = []
        for i in range(nb):
            if i == 0:
                lst = []
            elif i == nb - 1:
                lst = list(rng.permutation(nb))
            else:
                lst = list(rng.choice(nb, int(rng.integers(1, nb)), replace=False))
                lst += [lst[0]] * int(rng.integers(0, 2)) + [nb + 5, -1][: int(rng.integers(0, 3))]
                lst = lst[:nb]
                rng.shuffle(lst)
            counts[h, i] = len(lst) if i != nb - 1 else nb + 3
            idx[h, i, :len(lst)] = lst
            rows.append([j for j in lst if 0 <= j < nb])
        lists.append(rows)
    return counts, idx, lists


def _check_attn(name, tag, out, lse, want_o, want_l, dtype):
    tol_l2, tol_abs, tol_lse = ATTN_TOL[dtype]
    empty = np.isneginf(want_l)
    assert (np.isneginf(lse) == empty).all() and (out[empty] == 0).all()
    live = ~empty
    e = (rel_l2(out[live], want_o[live]), np.abs(out[live] - want_o[live]).max(),
         np.abs(lse[live] - want_l[live]).max())
    say(f"[gpu] cluster attention {name} {tag}: rel-l2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
    assert e[0] <= tol_l2 and e[1] <= tol_abs and e[2] <= tol_lse


@pytest.mark.parametrize("name", sorted(CASES))
def test_cluster_attention_matches_oracle(name):
    c = case(name)
    wl = c.wl
    cent, labels, sizes, order = clustered(c)
    lab = host(labels)
    cnt, ix, lists = _set_lists(wl.heads, wl.nblocks, host(sizes), 400 + sorted(CASES).index(name))
    out, lse = R.cluster_attn(c.q, c.k, c.v, sizes, order, torch.from_numpy(cnt).to(DEV),
                              torch.from_numpy(ix).to(DEV), c.p)
    o, l = host(out.float()).astype(np.float64), host(lse).astype(np.float64)
    for h in range(wl.heads):
        want_o, want_l = O.cluster_attention(c.q64[h], c.k64[h], c.v64[h], wl.block, lab[h], lists[h])
        _check_attn(name, f"set lists h={h}", o[h], l[h], want_o, want_l, wl.dtype)
    # the retrieval path: cluster scores -> top-p -> cluster attention
    S = R.score_clusters(c.q, cent, sizes, c.p)
    top_p = torch.full((wl.heads,), 0.9, dtype=torch.float32, device=DEV)
    _, counts, idx, dens = R.select_topp(S, top_p, c.p)
    out, lse = R.cluster_attn(c.q, c.k, c.v, sizes, order, counts, idx, c.p)
    o, l = host(out.float()).astype(np.float64), host(lse).astype(np.float64)
    cn, ixn = host(counts), host(idx)
    for h in range(wl.heads):
        sel = [ixn[h, i, :cn[h, i]] for i in range(wl.nblocks)]
        want_o, want_l = O.cluster_attention(c.q64[h], c.k64[h], c.v64[h], wl.block, lab[h], sel)
        _check_attn(name, f"top-p h={h} density {float(host(dens)[h]):.3f}", o[h], l[h], want_o, want_l, wl.dtype)


def test_contiguous_clusters_equal_block_attention():
    """Clusters that are the contiguous blocks (labels t // B): cluster
    attention on any list equals block-sparse attention on the same list."""
    c = case("bf16_d128_b64")
    clustered(c)
    wl, p = c.wl, c.p
    nb, b = wl.nblocks, wl.block
    sizes = torch.tensor([[min(b, wl.tokens - j * b) for j in range(nb)]] * wl.heads, dtype=torch.int32,
                         device=DEV)
    order = torch.arange(wl.tokens, dtype=torch.int32, device=DEV).repeat(wl.heads, 1).contiguous()
    cnt, ix, _ = _set_lists(wl.heads, nb, None, 450)
    cnt_t, ix_t = torch.from_numpy(cnt).to(DEV), torch.from_numpy(ix).to(DEV)
    o1, l1 = R.cluster_attn(c.q, c.k, c.v, sizes, order, cnt_t, ix_t, p)
    o2, l2 = R.block_sparse_attn(c.q, c.k, c.v, cnt_t, ix_t, p)
    torch.cuda.synchronize()
    a, bb = host(o1.float()).astype(np.float64), host(o2.float()).astype(np.float64)
    assert rel_l2(a, bb) <= 2e-3 and np.abs(a - bb).max() <= 1e-2
    la, lb = host(l1), host(l2)
    assert (np.isneginf(la) == np.isneginf(lb)).all()
    live = np.isfinite(lb)
    assert np.abs(la[live] - lb[live]).max() <= 1e-5


def test_cluster_attention_inconsistent_layout_stays_in_bounds():
    """Sizes that overrun the keys and token ids out of range: the call
    clamps them (results meaningless but finite, nothing written outside the
    outputs)."""
    c = case("bf16_d64_b64")
    wl, p = c.wl, c.p
    clustered(c)
    rng = np.random.default_rng(460)
    sizes = torch.from_numpy(rng.integers(-50, 4 * wl.tokens, (wl.heads, wl.nblocks)).astype(np.int32)).to(DEV)
    order = torch.from_numpy(rng.integers(-wl.tokens, 2 * wl.tokens, (wl.heads, wl.tokens)).astype(np.int32)).to(DEV)
    cnt = torch.full((wl.heads, wl.nblocks), wl.nblocks, dtype=torch.int32, device=DEV)
    ix = torch.arange(wl.nblocks, dtype=torch.int32, device=DEV).repeat(wl.heads, wl.nblocks, 1).contiguous()
    guard = torch.full((2, wl.heads, wl.tokens, wl.head_dim), 7.0, dtype=torch.bfloat16, device=DEV)
    out = guard[0]
    out, lse = R.cluster_attn(c.q, c.k, c.v, sizes, order, cnt, ix, p, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert (guard[1] == 7.0).all()
