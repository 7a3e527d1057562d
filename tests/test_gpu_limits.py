"""GPU checks at the largest problem the library accepts: 4096 blocks per
sequence.  One head, a 1 x 1 x T grid whose last block holds 20 tokens:

* 64-token blocks, head_dim 64: T = 4095 * 64 + 20 = 262,100 tokens (the
  attention's pair mode, the scorer's two blocks per workgroup);
* 128-token blocks, head_dim 128: T = 4095 * 128 + 20 = 524,180 tokens.

Scores of sampled query blocks against the fp64 oracle.  Attention on hand-made
lists: a full row (all 4096 blocks, shuffled), an empty row, the ragged last
block alone, a row with repeats and out-of-range entries, its pair partner
with a different list, a 3000-block row and short random rows elsewhere;
sampled rows against the oracle on the same (cleaned) lists; every row is
checked to be written, and empty exactly when its cleaned list is.
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
NB = 4096
TOL = (1e-2, 3e-2, 1e-3)        # bf16 attention bar: rel-L2, max abs, lse


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().cpu().numpy()


CASES = {
    # name: (head_dim, block)
    "b64_d64": (64, 64),
    "b128_d128": (128, 128),
}


def make_lists(rng, nb):
    counts = rng.integers(1, 65, size=nb).astype(np.int32)
    idx = np.zeros((nb, nb), np.int32)
    for i in range(nb):
        idx[i, :counts[i]] = rng.choice(nb, counts[i], replace=False)
    special = {
        0: rng.permutation(nb),                                  # full row, any order
        1: np.zeros(0, np.int64),                                # empty row
        2: np.array([nb - 1, 0, nb - 1, -1, nb, 9999]),          # repeats, out of range
        3: rng.choice(nb, 50, replace=False),                    # pair partner of row 2
        nb // 2 - 1: rng.choice(nb, 3000, replace=False),        # long row
        nb - 1: np.array([nb - 1]),                              # ragged block alone
    }
    for i, lst in special.items():
        counts[i] = len(lst)
        idx[i, :len(lst)] = lst
    return counts, idx, sorted(special) + [int(rng.integers(4, nb // 2 - 1))]


def clean(lst, nb):
    lst = np.asarray(lst)
    return np.unique(lst[(lst >= 0) & (lst < nb)])


@pytest.mark.parametrize("name", sorted(CASES))
def test_largest_problem(name):
    d, b = CASES[name]
    tokens = (NB - 1) * b + 20
    wl = W.Workload(300 + sorted(CASES).index(name), name, 1, (1, 1, tokens), d, b, "bf16", (0.9, 0.9, 0.9))
    assert wl.nblocks == NB
    say(f"[gpu] limits {name}: tokens={tokens} NB={NB} D={d} B={b}")
    inp = W.make_inputs(wl)
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    p = R.make_problem(q, wl.grid, wl.block)
    rng = np.random.default_rng(7 + b)

    S = R.score_blocks(q, k, p)
    counts, idx, rows = make_lists(rng, NB)
    # NaN-filled outputs: a row no workgroup writes (64-token blocks: a block
    # left out of every pair) keeps its NaN
    out0 = torch.full_like(q, float("nan"))
    lse0 = torch.full((1, tokens), float("nan"), dtype=torch.float32, device=DEV)
    out, lse = R.block_sparse_attn(q, k, v, torch.from_numpy(counts[None]).to(DEV),
                                   torch.from_numpy(idx[None]).to(DEV), p, out=out0, lse=lse0)
    torch.cuda.synchronize()
    # every row: written, and empty exactly when its list has no valid entry
    l_all = host(lse[0])
    assert not np.isnan(l_all).any() and not torch.isnan(out).any().item()
    has = np.array([clean(idx[i, :counts[i]], NB).size > 0 for i in range(NB)])
    assert (np.isneginf(l_all) == np.repeat(~has, b)[:tokens]).all()
    q64, k64, v64 = W.to_f64(inp.q[0]), W.to_f64(inp.k[0]), W.to_f64(inp.v[0])
    scale = 1.0 / np.sqrt(d)

    srows = [0, 1, NB // 2, NB - 2, NB - 1]
    s_or = O.score_head(q64, k64, b, scale, query_blocks=srows)
    ds = float(np.abs(host(S)[0, srows] - s_or).max())
    say(f"[gpu] limits {name}: scores of blocks {srows}: max |dS| {ds:.1e}")
    assert ds <= 1e-6

    lists = {i: clean(idx[i, :counts[i]], NB) for i in rows}
    o_or, l_or = O.block_sparse_attention(q64, k64, v64, b, lists, scale, query_blocks=rows)
    tr = np.concatenate([np.arange(i * b, min(tokens, (i + 1) * b)) for i in rows])
    o, l = host(out[0].float())[tr], host(lse[0])[tr]
    empty = np.isneginf(l_or)
    assert (np.isneginf(l) == empty).all() and (o[empty] == 0).all()
    assert empty.sum() == b       # exactly the empty row
    live = ~empty
    e = (rel_l2(o[live], o_or[live]), float(np.abs(o[live] - o_or[live]).max()),
         float(np.abs(l[live] - l_or[live]).max()))
    say(f"[gpu] limits {name}: attention rows {rows}: rel-l2 {e[0]:.2e} max-abs {e[1]:.2e} lse {e[2]:.2e}")
    assert e[0] <= TOL[0] and e[1] <= TOL[1] and e[2] <= TOL[2]
