"""GPU checks of the pair mode for 64-token bf16 blocks, where the library
pairs query blocks by the overlap of their key sets (a greedy matching in
segments of 128 blocks) and one workgroup walks the union of each pair.

Shape: 2 heads, NB = 2 * 128 + 1 = 257 blocks of 64 tokens (the last holds 20),
so the matching runs over two full segments and a last segment of one block,
which has no partner.  Hand-made lists stress the matching: runs of rows with
identical lists, rows with disjoint lists, empty rows, full rows in any order,
rows with repeats and out-of-range entries, and random rows elsewhere.
Outputs start as NaN, so a row that no workgroup writes fails; every row of
both heads is compared with the fp64 oracle on the same (cleaned) lists.
The omitted-key attention (the complement of every list) is checked the
same way.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import block_sparse_attention_scoring_amd as R
from parity import rel_l2

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = (1e-2, 3e-2, 1e-3)        # bf16 attention bar: rel-L2, max abs, lse
NB = 257


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().cpu().numpy()


def make_lists(rng, nb, h):
    counts = np.zeros(nb, np.int32)
    idx = np.zeros((nb, nb), np.int32)
    shared = rng.choice(nb, 40, replace=False)
    for i in range(nb):
        if 10 <= i < 30:                       # identical lists: pair at weight 0
            lst = shared
        elif 30 <= i < 60:                     # disjoint neighbours
            lst = np.arange(i % 4, nb, 4)[:50] if i % 2 else np.arange(2 + i % 4, nb, 4)[:50]
        elif i in (0, 128, 255):               # empty
            lst = np.zeros(0, np.int64)
        elif i in (1, 129, 256):               # full, shuffled
            lst = rng.permutation(nb)
        elif i == 2:                           # repeats and invalid entries
            lst = np.array([nb - 1, 0, nb - 1, -1, nb, 9999, 5, 5])
        else:
            lst = rng.choice(nb, int(rng.integers(1, 90)), replace=False)
        counts[i] = len(lst)
        idx[i, :len(lst)] = lst
    return counts, idx


def clean(lst, nb):
    lst = np.asarray(lst)
    return np.unique(lst[(lst >= 0) & (lst < nb)])


def check_all(tag, out, lse, lists, inp, wl):
    o_all, l_all = host(out.float()), host(lse)
    assert not np.isnan(o_all).any() and not np.isnan(l_all).any(), f"{tag}: unwritten rows"
    scale = 1.0 / np.sqrt(wl.head_dim)
    for h in range(wl.heads):
        q64, k64, v64 = W.to_f64(inp.q[h]), W.to_f64(inp.k[h]), W.to_f64(inp.v[h])
        o_or, l_or = O.block_sparse_attention(q64, k64, v64, wl.block, lists[h], scale)
        empty = np.isneginf(l_or)
        assert (np.isneginf(l_all[h]) == empty).all() and (o_all[h][empty] == 0).all()
        live = ~empty
        e = (rel_l2(o_all[h][live], o_or[live]), float(np.abs(o_all[h][live] - o_or[live]).max()),
             float(np.abs(l_all[h][live] - l_or[live]).max()))
        say(f"[gpu] pairs {tag} h={h}: every row, rel-l2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
        assert e[0] <= TOL[0] and e[1] <= TOL[1] and e[2] <= TOL[2]


@pytest.fixture(scope="module")
def case():
    tokens = (NB - 1) * 64 + 20
    wl = W.Workload(340, "pairs_257", 2, (1, 1, tokens), 128, 64, "bf16", (0.9, 0.9))
    assert wl.nblocks == NB
    say(f"[gpu] pairs: tokens={tokens} NB={NB} heads={wl.heads}")
    inp = W.make_inputs(wl)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    p = R.make_problem(q, wl.grid, wl.block)
    rng = np.random.default_rng(41)
    made = [make_lists(rng, NB, h) for h in range(wl.heads)]
    counts = torch.from_numpy(np.stack([c for c, _ in made])).to(DEV)
    idx = torch.from_numpy(np.stack([i for _, i in made])).to(DEV)
    lists = [[clean(i[r, :c[r]], NB) for r in range(NB)] for c, i in made]
    return wl, inp, q, k, v, p, counts, idx, lists


def test_pair_mode_every_row(case):
    wl, inp, q, k, v, p, counts, idx, lists = case
    out = torch.full_like(q, float("nan"))
    lse = torch.full((wl.heads, wl.tokens), float("nan"), dtype=torch.float32, device=DEV)
    R.block_sparse_attn(q, k, v, counts, idx, p, out=out, lse=lse)
    torch.cuda.synchronize()
    check_all("selected", out, lse, lists, inp, wl)


def test_pair_mode_omitted_every_row(case):
    wl, inp, q, k, v, p, counts, idx, lists = case
    out = torch.full_like(q, float("nan"))
    lse = torch.full((wl.heads, wl.tokens), float("nan"), dtype=torch.float32, device=DEV)
    R.attn_omitted(q, k, v, counts, idx, p, out=out, lse=lse)
    torch.cuda.synchronize()
    comp = [O.complement_lists(lists[h], NB) for h in range(wl.heads)]
    check_all("omitted", out, lse, comp, inp, wl)


def test_pair_mode_is_bitwise_repeatable(case):
    wl, inp, q, k, v, p, counts, idx, lists = case
    a, la = R.block_sparse_attn(q, k, v, counts, idx, p)
    b, lb = R.block_sparse_attn(q, k, v, counts, idx, p)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
