"""The Python binding rejects tensors the C entry points would misread.

The library takes bare pointers to dense row-major arrays, so a transposed
view, a wrong dtype or shape, or a host tensor must be refused on the host
before any library call.  These run on the CPU: every check fires before the
library is touched.
"""
import pytest
import torch

import block_sparse_attention_scoring_amd as R

H, N, D, BLK = 2, 192, 64, 64
NB = 3


def _prob(dtype=torch.bfloat16):
    q = torch.zeros(H, N, D, dtype=dtype)
    return R.make_problem(q, (3, 8, 8), BLK)


def _qkv(dtype=torch.bfloat16):
    return [torch.zeros(H, N, D, dtype=dtype) for _ in range(3)]


def test_host_tensors_are_refused():
    p = _prob()
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU tensor"):
        R.score_blocks(q, k, p)


def test_transposed_view_is_refused():
    p = _prob()
    q, k, _ = _qkv()
    kt = torch.zeros(H, D, N, dtype=torch.bfloat16).transpose(1, 2)     # [H, N, D] view, not row-major
    with pytest.raises(ValueError, match="contiguous"):
        R.score_blocks(q, kt, p)


def test_mixed_dtypes_are_refused():
    p = _prob()
    q, _, _ = _qkv()
    k32 = torch.zeros(H, N, D, dtype=torch.float32)
    with pytest.raises(TypeError, match="k must be torch.bfloat16"):
        R.score_blocks(q, k32, p)


def test_wrong_shapes_are_refused():
    p = _prob()
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="shape"):
        R.score_blocks(q[:, :128], k, p)
    counts = torch.zeros(H, NB, dtype=torch.int32)
    idx = torch.zeros(H, NB, NB + 1, dtype=torch.int32)
    with pytest.raises(ValueError, match="block_idx must have shape"):
        R.block_sparse_attn(q, k, v, counts, idx, p)


def test_selection_argument_types():
    p = _prob()
    s = torch.zeros(H, NB, NB, dtype=torch.float32)
    with pytest.raises(TypeError, match="top_p must be torch.float32"):
        R.select_topp(s, torch.full((H,), 0.9, dtype=torch.float64), p)
    with pytest.raises(TypeError, match="counts must be torch.int32"):
        R.select_topp(s, torch.full((H,), 0.9), p, counts=torch.zeros(H, NB, dtype=torch.int64))
    with pytest.raises(TypeError, match="head_active must be torch.uint8"):
        R.select_topp(s, torch.full((H,), 0.9), p, head_active=torch.ones(H, dtype=torch.bool))


def test_lists_and_outputs_of_attention():
    p = _prob()
    q, k, v = _qkv()
    counts = torch.zeros(H, NB, dtype=torch.int64)
    idx = torch.zeros(H, NB, NB, dtype=torch.int32)
    with pytest.raises(TypeError, match="counts must be torch.int32"):
        R.block_sparse_attn(q, k, v, counts, idx, p)
    counts = counts.int()
    with pytest.raises(TypeError, match="out must be torch.bfloat16"):
        R.block_sparse_attn(q, k, v, counts, idx, p, out=torch.zeros(H, N, D))
    with pytest.raises(ValueError, match="workspace"):
        R.block_sparse_attn(q, k, v, counts, idx, p, workspace=torch.zeros(16, dtype=torch.float32))


def test_drift_and_cluster_arguments():
    p = _prob()
    q, k, _ = _qkv()
    with pytest.raises(TypeError, match="q_ref must be torch.bfloat16"):
        R.mask_drift(q, k, q.float(), k, p, 0.05)
    with pytest.raises(ValueError, match="gram must have shape"):
        R.kmeans(k, torch.zeros(H, D, D + 1), p, iters=1)
    with pytest.raises(ValueError, match="sizes is required"):
        R.score_clusters(q, torch.zeros(H, NB, D), None, p)


def test_fp32_problem_takes_fp32_tensors():
    p = _prob(torch.float32)
    q, k, _ = _qkv(torch.bfloat16)
    with pytest.raises(TypeError, match="q must be torch.float32"):
        R.score_blocks(q, k, p)
