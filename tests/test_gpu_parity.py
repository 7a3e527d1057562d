"""GPU (gfx950) parity of the four library calls against the fp64 oracle.

Oracle-sized cases compare every output element; they span several tiles
of every kernel and end in a ragged block.  Acceptance:
  * block scores: |S_gpu - S_oracle| <= 1e-6 everywhere (rows sum to 1);
  * masks / lists / counts: bit-exact except tie rows (reported, tests/parity.py);
  * selection on identical fp32 scores: bit-exact, no exceptions;
  * attention (bf16 in, fp32 accumulate): rel-L2 <= 1e-2, max abs <= 3e-2;
    (fp32 in): rel-L2 <= 1e-4, max abs <= 1e-4; lse within 1e-3 (bf16) / 1e-4 (fp32);
  * drift: relative error <= 1e-6; refresh flags exact unless |d - tau| <= 1e-6.
Attention is compared on the GPU's own block lists, so mask ties cannot leak
into the attention check.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import block_sparse_attention_scoring_amd as R
from parity import check_rows, gpu_lists_from, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

ATTN_TOL = {"bf16": (1e-2, 3e-2, 1e-3), "fp32": (1e-4, 1e-4, 1e-4)}
S_TOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.to(DEV).contiguous()


def host(t):
    return t.detach().cpu().numpy()


CASES = {
    # name: (heads, grid, head_dim, block, dtype)
    "bf16_d128_b64": (2, (6, 20, 83), 128, 64, "bf16"),    # N=9960, NB=156, last block 40
    "bf16_d128_b128": (2, (6, 20, 83), 128, 128, "bf16"),  # NB=78, last block 104
    "bf16_d64_b128": (2, (5, 16, 51), 64, 128, "bf16"),    # N=4080, NB=32, last block 112
    "bf16_d64_b64": (3, (4, 9, 37), 64, 64, "bf16"),       # N=1332, NB=21, last block 52
    "bf16_d128_b128_short": (3, (2, 13, 31), 128, 128, "bf16"),  # N=806, NB=7, last block 38 (< 64)
    "bf16_d128_b128_even": (2, (5, 31, 81), 128, 128, "bf16"),  # N=12555, NB=99, last block 11 (4 chunks)
    "bf16_d128_b64_big": (1, (2, 140, 160), 128, 64, "bf16"),   # N=44800, NB=700 (two-pass scorer)
    "fp32_tiny": (1, (4, 8, 8), 64, 64, "fp32"),           # the tiny workload itself
    "fp32_d128_b128": (2, (3, 10, 29), 128, 128, "fp32"),  # N=870, NB=7, last block 102
}


def workload(name):
    if name == "fp32_tiny":
        return W.CONFIGS["tiny"]
    h, grid, d, b, dt = CASES[name]
    cid = 100 + sorted(CASES).index(name)
    return W.Workload(cid, name, h, grid, d, b, dt, (0.8, 0.9, 0.95))


class Run:
    """GPU path and oracle on one seeded case."""

    def __init__(self, name):
        wl = workload(name)
        self.wl = wl
        inp = W.make_inputs(wl)
        self.inp = inp
        self.q64, self.k64, self.v64 = W.to_f64(inp.q), W.to_f64(inp.k), W.to_f64(inp.v)
        say(f"[gpu] case {name}: heads={wl.heads} tokens={wl.tokens} D={wl.head_dim} "
            f"B={wl.block} NB={wl.nblocks} dtype={wl.dtype}")
        self.q, self.k, self.v = dev(inp.q), dev(inp.k), dev(inp.v)
        self.p = R.make_problem(self.q, wl.grid, wl.block)
        self.top_p = dev(torch.from_numpy(inp.top_p))
        self.S = R.score_blocks(self.q, self.k, self.p)
        self.mask, self.counts, self.idx, self.density = R.select_topp(self.S, self.top_p, self.p)
        self.out, self.lse = R.block_sparse_attn(self.q, self.k, self.v, self.counts, self.idx, self.p)
        torch.cuda.synchronize()
        self.S_or = O.score_blocks(self.q64, self.k64, wl.block)


_runs = {}


def run(name):
    if name not in _runs:
        _runs[name] = Run(name)
    return _runs[name]


@pytest.mark.parametrize("name", sorted(CASES))
def test_scores_match_oracle(name):
    r = run(name)
    s = host(r.S).astype(np.float64)
    err = np.abs(s - r.S_or).max()
    say(f"[gpu] {name}: max |dS| = {err:.3e}")
    assert err <= S_TOL
    np.testing.assert_allclose(s.sum(axis=-1), 1.0, atol=1e-5)
    csum_err = np.abs(np.cumsum(np.sort(s, -1)[..., ::-1], -1) - np.cumsum(np.sort(r.S_or, -1)[..., ::-1], -1)).max()
    assert csum_err < 1e-6


@pytest.mark.parametrize("name", sorted(CASES))
def test_selection_matches_oracle_with_ties_reported(name):
    r = run(name)
    wl = r.wl
    counts, idx, mask = host(r.counts), host(r.idx), host(r.mask)
    rows, srows, glists = [], [], []
    for h in range(wl.heads):
        lists = gpu_lists_from(counts[h], idx[h])
        for i in range(wl.nblocks):
            rows.append((h, i))
            srows.append(r.S_or[h, i])
            glists.append(lists[i])
            ind = np.zeros(wl.nblocks, np.uint8)
            ind[lists[i]] = 1
            assert (mask[h, i] == ind).all()
            assert (np.diff(lists[i]) > 0).all() and counts[h, i] >= 1
    res, ties, fails = check_rows(srows, r.inp.top_p, glists, rows)
    say(f"[gpu] {name}: rows {res}; tie rows {ties[:10]}{'...' if len(ties) > 10 else ''}")
    assert not fails, fails[:5]
    dens = host(r.density).astype(np.float64)
    np.testing.assert_allclose(dens, counts.reshape(wl.heads, -1).sum(-1) / wl.nblocks ** 2, rtol=1e-6)


@pytest.mark.parametrize("name", sorted(CASES))
def test_selection_on_identical_scores_is_exact(name):
    r = run(name)
    wl = r.wl
    s32 = r.S_or.astype(np.float32)
    mask, counts, idx, _ = R.select_topp(dev(torch.from_numpy(s32)), r.top_p, r.p)
    m_or, c_or, l_or = O.select_topp(s32.astype(np.float64), r.inp.top_p)
    assert (host(mask) == m_or).all() and (host(counts) == c_or).all()
    idx = host(idx)
    for h in range(wl.heads):
        for i in range(wl.nblocks):
            assert (idx[h, i, :c_or[h, i]] == l_or[h][i]).all()


@pytest.mark.parametrize("name", sorted(CASES))
def test_attention_matches_oracle_on_gpu_lists(name):
    r = run(name)
    wl = r.wl
    counts, idx = host(r.counts), host(r.idx)
    out = host(r.out.float()).astype(np.float64)
    lse = host(r.lse).astype(np.float64)
    tol_l2, tol_abs, tol_lse = ATTN_TOL[wl.dtype]
    worst = (0.0, 0.0, 0.0)
    for h in range(wl.heads):
        lists = gpu_lists_from(counts[h], idx[h])
        o_or, lse_or = O.block_sparse_attention(r.q64[h], r.k64[h], r.v64[h], wl.block, lists)
        e = (rel_l2(out[h], o_or), np.abs(out[h] - o_or).max(), np.abs(lse[h] - lse_or).max())
        worst = tuple(max(a, b) for a, b in zip(worst, e))
    say(f"[gpu] {name}: attention rel-L2 {worst[0]:.2e} max-abs {worst[1]:.2e} lse {worst[2]:.2e}")
    assert worst[0] <= tol_l2 and worst[1] <= tol_abs and worst[2] <= tol_lse


@pytest.mark.parametrize("name", ["bf16_d128_b128", "bf16_d64_b64", "fp32_d128_b128"])
def test_attention_lists_are_sets(name):
    """A row's list may come in any order, repeat blocks, hold entries
    outside [0, NB) and carry a count above NB: the visible keys are the set
    of valid listed blocks (oracle: token mask of that set), so the result
    equals the one on the sorted, duplicate-free lists bit for bit."""
    r = run(name)
    wl = r.wl
    nb = wl.nblocks
    counts, idx = host(r.counts), host(r.idx)
    rng = np.random.default_rng(7)
    c2 = counts.copy()
    i2 = np.zeros_like(idx)
    for h in range(wl.heads):
        for i in range(nb):
            sel = idx[h, i, :counts[h, i]]
            extra = list(rng.choice(sel, size=min(2, nb - len(sel)), replace=True)) if len(sel) else []
            if len(sel) + len(extra) < nb:
                extra.append(-3 if i % 2 else nb + 4)          # dropped entries
            row = np.concatenate([sel, np.asarray(extra, dtype=sel.dtype)])
            rng.shuffle(row)
            c2[h, i] = len(row)
            i2[h, i, :len(row)] = row
    # one row lists every block in reverse with a count above NB
    c2[0, 0] = nb + 3
    i2[0, 0] = np.arange(nb)[::-1]
    out, lse = R.block_sparse_attn(r.q, r.k, r.v, dev(torch.from_numpy(c2)), dev(torch.from_numpy(i2)), r.p)
    torch.cuda.synchronize()
    o_ref, l_ref = r.out, r.lse
    # row (0, 0) now sees every block: the oracle gives its reference
    o00, l00 = O.block_sparse_attention(r.q64[0], r.k64[0], r.v64[0], wl.block, [list(range(nb))],
                                        query_blocks=[0])
    out_h, lse_h = host(out.float()).astype(np.float64), host(lse).astype(np.float64)
    b = wl.block
    same = torch.equal(out[:, b:], o_ref[:, b:]) and torch.equal(out[1:], o_ref[1:])
    same_l = torch.equal(lse[:, b:], l_ref[:, b:]) and torch.equal(lse[1:], l_ref[1:])
    tol_l2, tol_abs, tol_lse = ATTN_TOL[wl.dtype]
    e = (rel_l2(out_h[0, :b], o00), np.abs(out_h[0, :b] - o00).max(), np.abs(lse_h[0, :b] - l00).max())
    say(f"[gpu] {name}: set-semantics rows bit-identical {same and same_l}; "
        f"all-blocks row rel-L2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
    assert same and same_l
    assert e[0] <= tol_l2 and e[1] <= tol_abs and e[2] <= tol_lse


@pytest.mark.parametrize("name", ["bf16_d128_b128", "bf16_d64_b64", "fp32_tiny"])
def test_drift_and_refresh_match_oracle(name):
    r = run(name)
    wl = r.wl
    inp = W.make_inputs(wl, keep_masters=True)
    q0, k0 = dev(inp.q), dev(inp.k)
    for s in (1, 2, 3):
        W.drift_step(inp, s)
    q1, k1 = dev(inp.q), dev(inp.k)
    d_or = O.drift(W.to_f64(inp.q), W.to_f64(inp.k), W.to_f64(q0.cpu()), W.to_f64(k0.cpu()))
    tau = float(np.median(d_or)) * (1 + 1e-3) if wl.heads > 1 else float(d_or[0]) * 0.5
    qr, kr = q0.clone(), k0.clone()
    d, f = R.mask_drift(q1, k1, qr, kr, r.p, tau, update_ref=True)
    d, f = host(d).astype(np.float64), host(f)
    say(f"[gpu] {name}: drift {d} oracle {d_or} tau {tau:.6g} refresh {f}")
    np.testing.assert_allclose(d, d_or, rtol=1e-6)
    want = O.refresh_decision(d_or, tau)
    tie = np.abs(d_or - float(np.float32(tau))) <= 1e-6
    assert ((f == want) | tie).all()
    for h in range(wl.heads):
        ref_q, ref_k = (q1[h], k1[h]) if f[h] else (q0[h], k0[h])
        assert torch.equal(qr[h], ref_q) and torch.equal(kr[h], ref_k)
    # identical inputs: zero drift, nothing refreshes
    d2, f2 = R.mask_drift(q1, k1, q1.clone(), k1.clone(), r.p, 0.0, update_ref=False)
    assert (host(d2) == 0).all() and (host(f2) == 0).all()


@pytest.mark.parametrize("name", ["bf16_d128_b64", "fp32_tiny"])
def test_bitwise_deterministic(name):
    r = run(name)
    S2 = R.score_blocks(r.q, r.k, r.p)
    m2, c2, i2, d2 = R.select_topp(S2, r.top_p, r.p)
    o2, l2 = R.block_sparse_attn(r.q, r.k, r.v, c2, i2, r.p)
    torch.cuda.synchronize()
    assert torch.equal(S2, r.S) and torch.equal(m2, r.mask) and torch.equal(c2, r.counts)
    assert torch.equal(o2, r.out) and torch.equal(l2, r.lse) and torch.equal(d2, r.density)


# ---------------------------------------------------------------- edge cases

def _problem_inputs(heads, grid, d, b, dtype=torch.bfloat16, seed=0):
    g = torch.Generator().manual_seed(seed)
    n = grid[0] * grid[1] * grid[2]
    q = torch.randn((heads, n, d), generator=g).to(dtype)
    k = torch.randn((heads, n, d), generator=g).to(dtype)
    v = torch.randn((heads, n, d), generator=g).to(dtype)
    return q, k, v


def test_zero_queries_uniform_scores_and_ceil_rule():
    say("[gpu] edge: zero queries")
    q, k, _ = _problem_inputs(2, (2, 10, 47), 128, 64)
    q.zero_()
    qd, kd = dev(q), dev(k)
    p = R.make_problem(qd, (2, 10, 47), 64)
    nb = p.nblocks
    S = host(R.score_blocks(qd, kd, p))
    np.testing.assert_allclose(S, 1.0 / nb, rtol=1e-6)
    tp = np.float32([0.33, 0.71])
    _, counts, idx, _ = R.select_topp(dev(torch.from_numpy(S)), dev(torch.from_numpy(tp)), p)
    counts, idx = host(counts), host(idx)
    for h in range(2):
        _, c_or, l_or = O.select_topp(S[h:h + 1].astype(np.float64), tp[h:h + 1])
        assert (counts[h] == c_or[0]).all()
        for i in range(nb):
            assert (idx[h, i, :counts[h, i]] == l_or[0][i]).all()


def test_single_block_problem():
    say("[gpu] edge: single block")
    q, k, v = _problem_inputs(1, (1, 2, 20), 64, 64)
    qd, kd, vd = dev(q), dev(k), dev(v)
    p = R.make_problem(qd, (1, 2, 20), 64)
    S = R.score_blocks(qd, kd, p)
    assert host(S).shape == (1, 1, 1) and abs(float(host(S)[0, 0, 0]) - 1.0) < 1e-6
    _, c, i, _ = R.select_topp(S, dev(torch.tensor([0.5])), p)
    out, lse = R.block_sparse_attn(qd, kd, vd, c, i, p)
    o_or, l_or = O.block_sparse_attention(W.to_f64(q[0]), W.to_f64(k[0]), W.to_f64(v[0]), 64, [[0]])
    assert rel_l2(host(out.float())[0], o_or) < 1e-2
    assert np.abs(host(lse)[0] - l_or).max() < 1e-3


def test_empty_rows_give_zero_and_neg_inf():
    say("[gpu] edge: empty rows")
    q, k, v = _problem_inputs(2, (2, 8, 24), 128, 128)
    qd, kd, vd = dev(q), dev(k), dev(v)
    p = R.make_problem(qd, (2, 8, 24), 128)
    nb = p.nblocks
    counts = torch.full((2, nb), nb, dtype=torch.int32)
    counts[0, 1] = 0
    counts[1, nb - 1] = 0
    idx = torch.arange(nb, dtype=torch.int32).repeat(2, nb, 1)
    out, lse = R.block_sparse_attn(qd, kd, vd, dev(counts), dev(idx), p)
    out, lse = host(out.float()), host(lse)
    assert (out[0, 128:256] == 0).all() and np.isneginf(lse[0, 128:256]).all()
    assert (out[1, (nb - 1) * 128:] == 0).all() and np.isneginf(lse[1, (nb - 1) * 128:]).all()
    o_or, _ = O.block_sparse_attention(W.to_f64(q[0]), W.to_f64(k[0]), W.to_f64(v[0]), 128,
                                       [list(range(nb))] * nb)
    assert rel_l2(out[0, :128], o_or[:128]) < 1e-2


def test_inactive_heads_are_left_untouched():
    say("[gpu] edge: head_active")
    q, k, _ = _problem_inputs(3, (2, 9, 40), 128, 64)
    qd, kd = dev(q), dev(k)
    p = R.make_problem(qd, (2, 9, 40), 64)
    nb = p.nblocks
    active = dev(torch.tensor([1, 0, 1], dtype=torch.uint8))
    S = torch.full((3, nb, nb), -7.0, device=DEV)
    R.score_blocks(qd, kd, p, head_active=active, out=S)
    Sh = host(S)
    assert (Sh[1] == -7.0).all() and (Sh[0] != -7.0).all() and (Sh[2] != -7.0).all()
    tp = dev(torch.full((3,), 0.9))
    mask = torch.full((3, nb, nb), 9, dtype=torch.uint8, device=DEV)
    counts = torch.full((3, nb), -1, dtype=torch.int32, device=DEV)
    idx = torch.full((3, nb, nb), -1, dtype=torch.int32, device=DEV)
    R.select_topp(S, tp, p, head_active=active, mask=mask, counts=counts, block_idx=idx)
    assert (host(mask)[1] == 9).all() and (host(counts)[1] == -1).all() and (host(idx)[1] == -1).all()
    assert (host(counts)[0] >= 1).all()


def test_max_blocks_cap_and_full_p():
    say("[gpu] edge: cap and p=1")
    rng = np.random.default_rng(5)
    nb = 300
    s = rng.dirichlet(np.full(nb, 0.2), size=(2, nb)).astype(np.float32)
    q = torch.zeros((2, nb * 64, 64), dtype=torch.bfloat16)
    p = R.make_problem(q, (1, 1, nb * 64), 64)
    sd = dev(torch.from_numpy(s))
    tp = np.float32([0.97, 1.0])
    mask, counts, idx, _ = R.select_topp(sd, dev(torch.from_numpy(tp)), p, max_blocks=17)
    m_or, c_or, l_or = O.select_topp(s.astype(np.float64), tp, max_blocks=17)
    assert (host(counts) == c_or).all() and (host(mask) == m_or).all()
    _, counts1, _, dens = R.select_topp(sd, dev(torch.ones(2)), p)
    assert (host(counts1) == nb).all() and np.allclose(host(dens), 1.0)


@pytest.mark.parametrize("nb", [1000, 2048, 4096])
def test_selection_large_rows(nb):
    say(f"[gpu] edge: selection NB={nb}")
    rng = np.random.default_rng(nb)
    rows = 24
    s = np.zeros((1, nb, nb), np.float32)
    s[0, :rows] = rng.dirichlet(np.full(nb, 0.05), size=rows)
    q = torch.zeros((1, nb * 64, 64), dtype=torch.bfloat16)
    p = R.make_problem(q, (1, 1, nb * 64), 64)
    mask, counts, idx, _ = R.select_topp(dev(torch.from_numpy(s)), dev(torch.tensor([0.9])), p)
    counts, idx = host(counts), host(idx)
    for i in range(rows):
        sel, kstar, _, _ = O.select_row(s[0, i].astype(np.float64), 0.9)
        assert counts[0, i] == kstar and (idx[0, i, :kstar] == sel).all()


def _rank_order_rows(nb, rng):
    """Rows whose rank-order fp64 running mass crosses p far from where the
    exact (or any reassociated) sum does: after 0.25 and 2^-25 - 2^-44 every
    3 * 2^-56 rounds the rank-order sum up by a whole ulp (2^-54), so it
    reaches p = 0.25 + 2^-25 after 1024 of them where the exact sum needs
    1366.  The tiny values are scattered over the row; a second row puts four
    2^-49 blocks ahead of them (rank-order count 902, exact 1201); in a third
    the first three blocks sum to p exactly (inclusive boundary)."""
    x, a = np.float32(3 * 2.0 ** -56), np.float32(2.0 ** -25 - 2.0 ** -44)
    rows = []
    r0 = np.zeros(nb, np.float32)
    r0[0], r0[1], r0[2:1800] = 0.25, a, x
    rows.append(r0)
    r1 = r0.copy()
    r1[1800:1804] = np.float32(2.0 ** -49)      # between a and x: taken before the tiny ones
    rows.append(r1)
    r2 = np.zeros(nb, np.float32)
    r2[0], r2[1], r2[2] = 0.25, np.float32(2.0 ** -25 - 2.0 ** -44), np.float32(2.0 ** -44)
    r2[3:600] = x                               # the prefix of three blocks is exactly p
    rows.append(r2)
    return [row[rng.permutation(nb)] for row in rows]


def test_selection_follows_rank_order_sum_near_threshold():
    """The selector's running mass is the fp64 sum in rank order (the
    oracle's definition), also where a reassociated sum would cross p at
    another rank: counts and lists equal the oracle's bit for bit."""
    nb = 2048
    say(f"[gpu] edge: rank-order running mass, NB={nb}")
    rng = np.random.default_rng(77)
    rows = _rank_order_rows(nb, rng)
    s = np.zeros((1, nb, nb), np.float32)
    for i, r in enumerate(rows):
        s[0, i] = r
    s[0, len(rows):len(rows) + 8] = rng.dirichlet(np.full(nb, 0.05), size=8)
    q = torch.zeros((1, nb * 64, 64), dtype=torch.bfloat16)
    p = R.make_problem(q, (1, 1, nb * 64), 64)
    pth = np.float32(0.25 + 2.0 ** -25)
    _, counts, idx, _ = R.select_topp(dev(torch.from_numpy(s)), dev(torch.tensor([pth])), p)
    counts, idx = host(counts), host(idx)
    for i in range(len(rows) + 8):
        sel, kstar, _, csum = O.select_row(s[0, i].astype(np.float64), float(pth))
        assert counts[0, i] == kstar and (idx[0, i, :kstar] == sel).all(), (i, int(counts[0, i]), kstar)
    # the constructed rows do need the rank order: an exact sum would keep more blocks
    assert O.select_row(s[0, 0].astype(np.float64), float(pth))[1] == 1026
