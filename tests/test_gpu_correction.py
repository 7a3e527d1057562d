"""RECAP's cached correction on the GPU against the oracle.

RECAP (Reciprocal Sparse Attention and Hierarchical Caching for Efficient
Video Diffusion), Abstract: a dense refinement over the interactions that
sparse attention omits is cached and corrects later sparse outputs, weighted
by the fresh sparse statistics.

* rsa_attn_omitted against the oracle's omitted_attention, on lists read as
  sets (shuffled, repeated, out-of-range entries, over-long counts, empty and
  full rows), both dtypes, ragged last blocks;
* rsa_attn_merge of the GPU's own sparse and omitted parts against dense
  attention (the oracle's merge identity), and against the oracle's merge of
  the same parts;
* rsa_block_sparse_attn_corrected (the sparse pass joined with the cached
  part inside the attention kernel) against dense attention, against the
  GPU's sparse pass followed by rsa_attn_merge, and in place;
* heads switched off by head_active keep their cached rows bit for bit;
* the mask cache with the correction on, over a drifting trajectory (q, k and
  v walk), against the oracle's corrected_trajectory, and after a Turbo
  re-selection (every head's omitted part recomputed).
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import block_sparse_attention_scoring_amd as R
from parity import classify_row, rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (rel L2, max abs) on outputs of magnitude ~1, max abs on lse
ATTN_TOL = {"bf16": (1e-2, 3e-2, 1e-3), "fp32": (1e-4, 1e-4, 1e-4)}

CASES = {
    # name: (heads, grid, head_dim, block, dtype)
    "bf16_d128_b128": (2, (6, 20, 83), 128, 128, "bf16"),  # N=9960, NB=78, last block 104
    "bf16_d128_b64": (2, (3, 10, 41), 128, 64, "bf16"),    # N=1230, NB=20, last block 14
    "bf16_d64_b64": (3, (4, 9, 37), 64, 64, "bf16"),       # N=1332, NB=21, last block 52
    "fp32_d128_b128": (2, (3, 10, 29), 128, 128, "fp32"),  # N=870, NB=7, last block 102
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def workload(name):
    h, grid, d, b, dt = CASES[name]
    return W.Workload(200 + sorted(CASES).index(name), name, h, grid, d, b, dt, (0.8, 0.9, 0.95))


def set_lists(heads, nb, seed):
    """Row lists as sets in the library's layout: counts [H, NB], idx [H, NB, NB].

    Returns (counts, idx, python lists per head and row)."""
    rng = np.random.default_rng(seed)
    counts = np.zeros((heads, nb), np.int32)
    idx = np.full((heads, nb, nb), -1, np.int32)
    lists = []
    for h in range(heads):
        rows = []
        for i in range(nb):
            if i == 0:
                lst = []                                     # nothing listed: all omitted
            elif i == nb - 1:
                lst = list(rng.permutation(nb))              # everything listed: nothing omitted
            else:
                c = int(rng.integers(1, nb))
                lst = list(rng.choice(nb, c, replace=False))
                lst += [lst[0]] * int(rng.integers(0, 2))    # a repeat
                lst += [nb + 7, -3][: int(rng.integers(0, 3))]  # ignored entries
                lst = lst[:nb]
                rng.shuffle(lst)
            counts[h, i] = len(lst) if i != nb - 1 else nb + 9   # over-long count clamps to NB
            idx[h, i, :len(lst)] = lst
            rows.append([j for j in lst if 0 <= j < nb])
        lists.append(rows)
    return counts, idx, lists


class Case:
    def __init__(self, name):
        wl = workload(name)
        self.wl = wl
        inp = W.make_inputs(wl)
        self.q64, self.k64, self.v64 = W.to_f64(inp.q), W.to_f64(inp.k), W.to_f64(inp.v)
        say(f"[gpu] correction case {name}: heads={wl.heads} tokens={wl.tokens} D={wl.head_dim} "
            f"B={wl.block} NB={wl.nblocks} dtype={wl.dtype}")
        self.q, self.k, self.v = (t.to(DEV).contiguous() for t in (inp.q, inp.k, inp.v))
        self.p = R.make_problem(self.q, wl.grid, wl.block)
        c, ix, self.lists = set_lists(wl.heads, wl.nblocks, 300 + wl.cid)
        self.counts = torch.from_numpy(c).to(DEV)
        self.idx = torch.from_numpy(ix).to(DEV)
        self.o_out, self.o_lse = R.attn_omitted(self.q, self.k, self.v, self.counts, self.idx, self.p)
        self.s_out, self.s_lse = R.block_sparse_attn(self.q, self.k, self.v, self.counts, self.idx, self.p)
        self.parts = (host(self.s_out), host(self.s_lse), host(self.o_out), host(self.o_lse))
        self.m_out, self.m_lse = self.s_out.clone(), self.s_lse.clone()
        R.attn_merge(self.m_out, self.m_lse, self.o_out, self.o_lse, self.p)
        self.c_out, self.c_lse = R.block_sparse_attn_corrected(self.q, self.k, self.v, self.counts, self.idx,
                                                               self.o_out, self.o_lse, self.p)
        torch.cuda.synchronize()


_cases = {}


def case(name):
    if name not in _cases:
        _cases[name] = Case(name)
    return _cases[name]


@pytest.mark.parametrize("name", sorted(CASES))
def test_omitted_attention_matches_oracle(name):
    c = case(name)
    wl = c.wl
    tol_l2, tol_abs, tol_lse = ATTN_TOL[wl.dtype]
    out, lse = host(c.o_out), host(c.o_lse)
    b, nb = wl.block, wl.nblocks
    for h in range(wl.heads):
        o_or, l_or = O.omitted_attention(c.q64[h], c.k64[h], c.v64[h], b, c.lists[h])
        empty = np.isneginf(l_or)
        assert (np.isneginf(lse[h]) == empty).all()
        assert (out[h][empty] == 0).all()
        assert empty[(nb - 1) * b:].all() and not empty[:b].any()
        live = ~empty
        e = (rel_l2(out[h][live], o_or[live]), np.abs(out[h][live] - o_or[live]).max(),
             np.abs(lse[h][live] - l_or[live]).max())
        say(f"[gpu] omitted {name} h={h}: rel-l2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
        assert e[0] <= tol_l2 and e[1] <= tol_abs and e[2] <= tol_lse


@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_merged_with_omitted_is_dense(name):
    c = case(name)
    wl = c.wl
    tol_l2, tol_abs, tol_lse = ATTN_TOL[wl.dtype]
    out, lse = host(c.m_out), host(c.m_lse)
    full = [list(range(wl.nblocks))] * wl.nblocks
    for h in range(wl.heads):
        o_or, l_or = O.block_sparse_attention(c.q64[h], c.k64[h], c.v64[h], wl.block, full)
        e = (rel_l2(out[h], o_or), np.abs(out[h] - o_or).max(), np.abs(lse[h] - l_or).max())
        say(f"[gpu] merged vs dense {name} h={h}: rel-l2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
        assert e[0] <= tol_l2 and e[1] <= tol_abs and e[2] <= tol_lse


@pytest.mark.parametrize("name", sorted(CASES))
def test_merge_matches_oracle_merge_of_same_parts(name):
    """The merge alone: the oracle joins the very parts the GPU joined (their
    stored values), so the only difference left is the merge's own fp32
    arithmetic and, for bf16, the final rounding (half a unit in the last
    place of an 8-bit significand: at most 2^-8 relative)."""
    c = case(name)
    so, sl, oo, ol = c.parts
    o_or, l_or = O.merge_partial(so.reshape(-1, so.shape[-1]), sl.reshape(-1),
                                 oo.reshape(-1, oo.shape[-1]), ol.reshape(-1))
    out, lse = host(c.m_out).reshape(o_or.shape), host(c.m_lse).reshape(-1)
    rel = 2.0 ** -8 if c.wl.dtype == "bf16" else 0.0
    parts = np.abs(so).reshape(o_or.shape).max(axis=1, keepdims=True) + \
        np.abs(oo).reshape(o_or.shape).max(axis=1, keepdims=True)
    err = np.abs(out - o_or) - (rel * np.abs(o_or) + 1e-6 * parts)
    say(f"[gpu] merge {name}: worst excess over the bound {err.max():.2e}")
    assert (err <= 0).all()
    assert (np.isneginf(lse) == np.isneginf(l_or)).all()
    live = np.isfinite(l_or)
    assert np.abs(lse[live] - l_or[live]).max() <= 2e-6 * max(1.0, np.abs(l_or[live]).max())


@pytest.mark.parametrize("name", sorted(CASES))
def test_corrected_attention_is_dense(name):
    """Sparse pass and cached omitted part joined in the attention kernel: on
    the inputs the part was cached from, the union of the two key sets is every
    key, so the result is dense attention."""
    c = case(name)
    wl = c.wl
    tol_l2, tol_abs, tol_lse = ATTN_TOL[wl.dtype]
    out, lse = host(c.c_out), host(c.c_lse)
    full = [list(range(wl.nblocks))] * wl.nblocks
    for h in range(wl.heads):
        o_or, l_or = O.block_sparse_attention(c.q64[h], c.k64[h], c.v64[h], wl.block, full)
        e = (rel_l2(out[h], o_or), np.abs(out[h] - o_or).max(), np.abs(lse[h] - l_or).max())
        say(f"[gpu] corrected vs dense {name} h={h}: rel-l2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
        assert e[0] <= tol_l2 and e[1] <= tol_abs and e[2] <= tol_lse


@pytest.mark.parametrize("name", sorted(CASES))
def test_corrected_matches_sparse_then_merge(name):
    """One pass against two: the fused join takes the sparse output before its
    rounding to the output type.  bf16 rounds to nearest with an 8-bit
    significand (error at most 2^-8 relative), so the two differ by at most
    that rounding of the sparse part plus one rounding of each result; fp32
    by a few fp32 roundings.  The lse is the same."""
    c = case(name)
    out, m_out = host(c.c_out), host(c.m_out)
    so = np.abs(host(c.s_out)).max(axis=-1, keepdims=True)
    oo = np.abs(host(c.o_out)).max(axis=-1, keepdims=True)
    if c.wl.dtype == "bf16":
        bound = 2.0 ** -7 * np.maximum(np.abs(out), np.abs(m_out)) + 2.0 ** -8 * so + 1e-6 * oo
    else:
        bound = 1e-6 * (so + oo)
    excess = np.abs(out - m_out) - bound
    say(f"[gpu] corrected vs sparse + merge {name}: worst excess over the bound {excess.max():.2e}")
    assert (excess <= 0).all()
    lse, m_lse = host(c.c_lse), host(c.m_lse)
    assert (np.isneginf(lse) == np.isneginf(m_lse)).all()
    live = np.isfinite(m_lse)
    assert np.abs(lse[live] - m_lse[live]).max() <= 2e-6 * max(1.0, np.abs(m_lse[live]).max())


def test_corrected_in_place():
    """out and lse may be the cached part itself: the same result, bit for bit."""
    c = case("bf16_d128_b64")
    out, lse = c.o_out.clone(), c.o_lse.clone()
    R.block_sparse_attn_corrected(c.q, c.k, c.v, c.counts, c.idx, out, lse, c.p, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, c.c_out) and torch.equal(lse, c.c_lse)


def test_merge_with_empty_parts_is_exact():
    """A part with lse = -inf has weight 0: the other part comes through bit for
    bit; two empty parts give zero rows and -inf."""
    c = case("bf16_d64_b64")
    out, lse = c.s_out.clone(), c.s_lse.clone()
    none_out = torch.full_like(out, 3.0)
    none_lse = torch.full_like(lse, float("-inf"))
    R.attn_merge(out, lse, none_out, none_lse, c.p)
    e_out, e_lse = torch.zeros_like(out), torch.full_like(lse, float("-inf"))
    R.attn_merge(e_out, e_lse, none_out, none_lse, c.p)
    torch.cuda.synchronize()
    live = torch.isfinite(c.s_lse)
    assert torch.equal(out[live], c.s_out[live]) and torch.equal(lse, c.s_lse)
    assert (e_out == 0).all() and torch.isneginf(e_lse).all()


def test_inactive_heads_keep_their_cache():
    c = case("bf16_d64_b64")
    active = torch.tensor([0, 1, 0], dtype=torch.uint8, device=DEV)
    out = torch.full_like(c.o_out, 7.0)
    lse = torch.full_like(c.o_lse, 5.0)
    R.attn_omitted(c.q, c.k, c.v, c.counts, c.idx, c.p, head_active=active, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (out[0] == 7.0).all() and (out[2] == 7.0).all()
    assert (lse[0] == 5.0).all() and (lse[2] == 5.0).all()
    assert torch.equal(out[1], c.o_out[1]) and torch.equal(lse[1], c.o_lse[1])


def test_corrected_trajectory_against_oracle():
    """Mask cache with the correction on over 5 steps of a drifting 3-head case.

    q, k and v take the workload generator's random walk; the drift threshold
    is set so that heads refresh at different steps.  Per step: refresh flags
    equal the oracle's (unless the drift sits within 1e-6 of the threshold),
    lists equal the oracle's or differ on reported tie rows only, and the
    corrected output matches the oracle's corrected output on every query
    block whose list agrees."""
    wl = W.Workload(250, "corr_traj", 3, (4, 9, 37), 64, 64, "bf16", (0.8, 0.9, 0.95))
    tau = 0.012
    inp = W.make_inputs(wl, keep_masters=True)
    q = inp.q.to(DEV)
    p = R.make_problem(q, wl.grid, wl.block)
    cache = R.MaskCache(p, torch.from_numpy(inp.top_p).to(DEV), tau, correction=True)
    steps64, gpu = [], []
    for s in range(5):
        if s > 0:
            W.drift_step(inp, s, values=True)
        say(f"[gpu] corrected trajectory step {s}")
        q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
        out, lse = cache.step(q, k, v)
        torch.cuda.synchronize()
        refresh = cache.refresh.cpu().numpy() if s > 0 else np.ones(wl.heads, np.uint8)
        gpu.append((refresh.copy(), cache.counts.cpu().numpy(), cache.block_idx.cpu().numpy(),
                    host(out), host(lse), cache.drift.cpu().numpy().astype(np.float64)))
        steps64.append((W.to_f64(inp.q), W.to_f64(inp.k), W.to_f64(inp.v)))
    tol_l2, tol_abs, tol_lse = ATTN_TOL["bf16"]
    refreshes = np.zeros(wl.heads, int)
    b, nb = wl.block, wl.nblocks
    scale = 1.0 / np.sqrt(wl.head_dim)
    for s, (ref, g) in enumerate(zip(O.corrected_trajectory(steps64, b, inp.top_p, tau), gpu)):
        r_or, lists_or, o_or, l_or, _, _ = ref
        r_g, cnt, ix, o_g, l_g, d_g = g
        if s > 0:
            d_or = O.drift(steps64[s][0], steps64[s][1], *_snapshots(steps64, gpu, s))
            near = np.abs(d_or - float(np.float32(tau))) <= 1e-6
            assert ((r_g == r_or) | near).all(), (s, r_g, r_or, d_or)
            if not (r_g == r_or).all():
                pytest.skip(f"refresh differs at step {s} on a threshold tie")
        refreshes += r_g
        for h in range(wl.heads):
            ok_rows = []
            s_head = None
            for i in range(nb):
                g_list = sorted(ix[h, i, :cnt[h, i]].tolist())
                if g_list == [int(j) for j in lists_or[h][i]]:
                    ok_rows.append(i)
                    continue
                if s_head is None:
                    last = max(t for t in range(s + 1) if gpu[t][0][h])
                    s_head = O.score_head(steps64[last][0][h], steps64[last][1][h], b, scale)
                kind, _ = classify_row(s_head[i], float(inp.top_p[h]), g_list)
                assert kind == "tie", (s, h, i)
                say(f"[gpu] step {s} head {h} row {i}: tie row, output not compared")
            rows = np.concatenate([np.arange(*O.block_bounds(i, wl.tokens, b)) for i in ok_rows])
            e = (rel_l2(o_g[h][rows], o_or[h][rows]), np.abs(o_g[h][rows] - o_or[h][rows]).max(),
                 np.abs(l_g[h][rows] - l_or[h][rows]).max())
            say(f"[gpu] corrected step {s} h={h}: rel-l2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
            assert e[0] <= tol_l2 and e[1] <= tol_abs and e[2] <= tol_lse
    say(f"[gpu] corrected trajectory refreshes per head: {refreshes.tolist()}")
    assert (refreshes > 1).any() and (refreshes < 5).any()   # heads refresh at different steps


def test_turbo_then_corrected_step_is_dense():
    """A Turbo re-selection changes every head's list, so the next corrected
    step recomputes every head's omitted part: on unchanged inputs (no head
    refreshes) the corrected output is still dense attention."""
    c = case("bf16_d64_b64")
    wl = c.wl
    cache = R.MaskCache(c.p, torch.from_numpy(wl.top_p_array()).to(DEV), 0.05, correction=True)
    cache.step(c.q, c.k, c.v)
    before = cache.counts.clone()
    cache.turbo(torch.full((wl.heads,), 0.6, dtype=torch.float32, device=DEV))
    out, lse = cache.step(c.q, c.k, c.v)
    torch.cuda.synchronize()
    assert int(cache.refresh.sum().item()) == 0                      # nothing refreshed by drift
    assert (cache.counts <= before).all() and (cache.counts < before).any()  # Turbo shrank the lists
    tol_l2, tol_abs, tol_lse = ATTN_TOL["bf16"]
    o, l = host(out), host(lse)
    full = [list(range(wl.nblocks))] * wl.nblocks
    for h in range(wl.heads):
        o_or, l_or = O.block_sparse_attention(c.q64[h], c.k64[h], c.v64[h], wl.block, full)
        e = (rel_l2(o[h], o_or), np.abs(o[h] - o_or).max(), np.abs(l[h] - l_or).max())
        say(f"[gpu] turbo + corrected h={h}: rel-l2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
        assert e[0] <= tol_l2 and e[1] <= tol_abs and e[2] <= tol_lse


def _snapshots(steps64, gpu, s):
    """Each head's (q, k) at its last refresh before step s, stacked [H, N, D]."""
    heads = steps64[0][0].shape[0]
    qs, ks = [], []
    for h in range(heads):
        last = max(t for t in range(s) if gpu[t][0][h])
        qs.append(steps64[last][0][h])
        ks.append(steps64[last][1][h])
    return np.stack(qs), np.stack(ks)
