"""The hot path inside a HIP graph.

The library's calls only enqueue kernels on the caller's stream: no device
allocation, copy, memset or synchronisation.  So one step (drift, scoring,
top-p selection, attention) can be captured once and replayed.  The step is
captured with every buffer (outputs and workspaces) allocated beforehand and
replayed several times, with the outputs overwritten and other eager library
work run between replays; every replay must equal the eager step bit for bit.
Both attention modes are covered: 128-token blocks, and 64-token blocks in
pairs (the pairing kernels run inside the graph too).
"""
import sys

import pytest
import torch

import workloads as W
import block_sparse_attention_scoring_amd as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    # name: (heads, grid, head_dim, block)
    "b128": (3, (3, 12, 29), 128, 128),   # N=1044, NB=9, last block 20
    "b64": (3, (4, 9, 37), 128, 64),      # N=1332, NB=21 (pairs, one block alone)
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Step:
    """Every buffer of one step, allocated before any capture."""

    def __init__(self, name):
        h, grid, d, b = CASES[name]
        wl = W.Workload(360 + sorted(CASES).index(name), name, h, grid, d, b, "bf16", (0.8, 0.9, 0.95))
        inp = W.make_inputs(wl)
        self.q, self.k, self.v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
        self.q_ref, self.k_ref = self.q.clone(), self.k.clone()
        self.p = p = R.make_problem(self.q, wl.grid, wl.block)
        self.tp = torch.from_numpy(inp.top_p).to(DEV)
        nb = p.nblocks
        f = dict(device=DEV)
        self.S = torch.empty((h, nb, nb), dtype=torch.float32, **f)
        self.mask = torch.empty((h, nb, nb), dtype=torch.uint8, **f)
        self.counts = torch.empty((h, nb), dtype=torch.int32, **f)
        self.idx = torch.empty((h, nb, nb), dtype=torch.int32, **f)
        self.dens = torch.empty((h,), dtype=torch.float32, **f)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((h, wl.tokens), dtype=torch.float32, **f)
        self.drift = torch.empty((h,), dtype=torch.float32, **f)
        self.refresh = torch.empty((h,), dtype=torch.uint8, **f)
        ws = lambda op: torch.empty(max(R.workspace_bytes(p, op), 1), dtype=torch.uint8, **f)
        self.ws_s, self.ws_a, self.ws_d = ws(R.OP_SCORE), ws(R.OP_ATTN), ws(R.OP_DRIFT)

    def run(self):
        R.mask_drift(self.q, self.k, self.q_ref, self.k_ref, self.p, 0.05, update_ref=False,
                     drift=self.drift, refresh=self.refresh, workspace=self.ws_d)
        R.score_blocks(self.q, self.k, self.p, out=self.S, workspace=self.ws_s)
        R.select_topp(self.S, self.tp, self.p, mask=self.mask, counts=self.counts, block_idx=self.idx,
                      density=self.dens)
        R.block_sparse_attn(self.q, self.k, self.v, self.counts, self.idx, self.p, out=self.out, lse=self.lse,
                            workspace=self.ws_a)

    def results(self):
        # block_idx is defined only in each row's first counts[h, I] entries
        valid = torch.arange(self.idx.shape[-1], device=DEV) < self.counts[..., None]
        return [t.clone() for t in (self.S, self.mask, self.counts, torch.where(valid, self.idx, -1), self.dens,
                                    self.out, self.lse, self.drift, self.refresh)]

    def scribble(self):
        for t in (self.S, self.dens, self.lse, self.drift):
            t.fill_(float("nan"))
        self.out.fill_(float("nan"))
        for t in (self.mask, self.counts, self.idx, self.refresh):
            t.fill_(7)


@pytest.mark.parametrize("name", sorted(CASES))
def test_step_replays_from_a_hip_graph(name):
    st = Step(name)
    say(f"[gpu] graph {name}: eager step")
    st.run()
    torch.cuda.synchronize()
    want = st.results()
    # warm up on a side stream, then capture on it
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()
    other = Step(name)   # eager library work between replays, on its own buffers
    for rep in range(4):
        st.scribble()
        other.run()
        torch.cuda.synchronize()
        say(f"[gpu] graph {name}: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got = st.results()
        for a, b in zip(want, got):
            assert torch.equal(a, b) or (a.is_floating_point() and torch.equal(a.nan_to_num(), b.nan_to_num())
                                         and torch.equal(a.isnan(), b.isnan())), f"replay {rep} differs"
