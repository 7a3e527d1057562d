"""rsa_score_blocks_noalloc through the C ABI against rsa_score_blocks.

The allocation-free entry point runs the same kernels with the library's
static device array as the workspace, so its scores must equal those of the
regular call bit for bit.  Two calls in a row, the second on a smaller
problem (the array keeps the first call's contents); a problem whose
workspace exceeds the array is rejected before any launch and leaves the
output untouched.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import workloads as W
import block_sparse_attention_scoring_amd as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _call_noalloc(q, k, p, out, head_active=None):
    lib = R.lib()
    st = lib.rsa_score_blocks_noalloc(ctypes.byref(p), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                      None if head_active is None else ctypes.c_void_p(head_active.data_ptr()),
                                      ctypes.c_void_p(out.data_ptr()),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("shape", [
    # (heads, grid, block): a large call, then a smaller one on the same array
    [(6, (7, 20, 64), 128), (2, (3, 11, 29), 128)],
    [(3, (5, 24, 60), 64), (1, (2, 9, 17), 64)],
])
def test_noalloc_scores_equal_regular_call(shape):
    for i, (heads, grid, block) in enumerate(shape):
        wl = W.Workload(300 + i, f"noalloc{i}", heads, grid, 128, block, "bf16", (0.9,))
        say(f"[gpu] noalloc call {i}: heads={heads} grid={grid} block={block} NB={wl.nblocks}")
        inp = W.make_inputs(wl)
        q, k = inp.q.to(DEV), inp.k.to(DEV)
        p = R.make_problem(q, wl.grid, wl.block)
        want = R.score_blocks(q, k, p)
        got = torch.full_like(want, float("nan"))
        assert _call_noalloc(q, k, p, got) == 0
        torch.cuda.synchronize()
        assert torch.equal(got, want), float((got - want).abs().max())
        # through the Python binding too, with an inactive head left untouched
        act = torch.ones(heads, dtype=torch.uint8, device=DEV)
        act[0] = 0
        keep = torch.full_like(want, 7.0)
        R.score_blocks_noalloc(q, k, p, head_active=act, out=keep)
        torch.cuda.synchronize()
        assert torch.equal(keep[1:], want[1:]) and bool((keep[0] == 7.0).all())


def test_noalloc_rejects_problems_beyond_the_array():
    # 64 heads x 4096 blocks of 64: the workspace is far above 64 MiB; the
    # call fails on the host, so small stand-in buffers are never read
    p = R.Problem(64, 4096 * 64, 64, 1, 64, 4096, 64, R.RSA_BF16, 0.0)
    q = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    need = R.workspace_bytes(p, R.OP_SCORE)
    assert need > 64 * 2 ** 20
    out = torch.full((1,), 3.0, device=DEV)   # never written: the call fails first
    assert _call_noalloc(q, q, p, out) == 5    # RSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(out[0]) == 3.0
