"""The C-ABI library loads, exports every declared symbol and validates on the host.

No call here reaches a kernel launch: every case fails validation, which
runs before anything is enqueued, so these tests need no GPU.  Host memory
passed in place of device buffers shows that a rejected call writes nothing.
"""
import ctypes

import numpy as np
import pytest

import block_sparse_attention_scoring_amd as R
from block_sparse_attention_scoring_amd import binding as B

OK, NULL, SHAPE, DTYPE, ALIGN, WS, HIP, ARG = range(8)


def prob(heads=2, grid=(4, 8, 8), d=128, b=64, dtype=0, scale=0.0):
    f, y, x = grid
    return B.Problem(heads, f * y * x, d, f, y, x, b, dtype, scale)


@pytest.fixture(scope="module")
def lib():
    return R.lib()


class Buf:
    """Host buffer standing in for a device pointer; must stay untouched."""

    def __init__(self, nbytes=4096, fill=0x5A):
        self.a = np.full(nbytes + 512, fill, np.uint8)
        off = (-self.a.ctypes.data) % 256
        self.view = self.a[off:off + nbytes]
        self.ptr = ctypes.c_void_p(self.view.ctypes.data)

    def untouched(self):
        return bool((self.a == 0x5A).all())


def test_exports_every_declared_symbol(lib):
    names = R.declared_functions()
    assert set(names) == {"rsa_workspace_bytes", "rsa_status_str", "rsa_version", "rsa_score_blocks",
                          "rsa_select_topp", "rsa_mask_drift", "rsa_block_sparse_attn",
                          "rsa_dense_block_mass", "rsa_score_blocks_pooled", "rsa_attn_omitted",
                          "rsa_attn_merge", "rsa_block_sparse_attn_corrected", "rsa_query_gram", "rsa_kmeans",
                          "rsa_score_clusters", "rsa_cluster_attn", "rsa_score_blocks_noalloc"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.rsa_version() == 10000
    names = [lib.rsa_status_str(i).decode() for i in range(8)]
    assert names == ["RSA_OK", "RSA_ERR_NULL", "RSA_ERR_SHAPE", "RSA_ERR_DTYPE", "RSA_ERR_ALIGN",
                     "RSA_ERR_WORKSPACE", "RSA_ERR_HIP", "RSA_ERR_ARG"]
    assert lib.rsa_status_str(99) == b"unknown"


def test_workspace_sizes():
    p = prob(heads=40, grid=(21, 45, 80), b=128)           # 75600 tokens, 591 blocks
    nbp = 608
    al = lambda x: -(-x // 256) * 256
    want = al(4 * 40 * 591 * 128) + al(4 * 40 * 591) + 2 * al(2 * 40 * nbp * 128) + al(4 * 40)
    assert B.workspace_bytes(p, B.OP_SCORE) == want
    assert B.workspace_bytes(p, B.OP_DRIFT) == 8 * 2 * 64 * 40
    assert B.workspace_bytes(p, B.OP_SELECT) == 0
    # attention: v re-laid out key-major (bf16), then the canonical list
    # counts and lists of every row, then (bf16) the dispatch order
    lists = al(4 * 40 * 591) + al(4 * 40 * 591 * 591)
    # 40 heads of 38.7 MB (K + V^T) in 10 groups of 4: 8 eighths of ceil(4 * 591 / 8) units
    order = al(4 * 8 * 10 * 296)
    assert B.workspace_bytes(p, B.OP_ATTN) == al(2 * 40 * 128 * 591 * 128) + lists + order
    assert B.workspace_bytes(prob(heads=40, grid=(21, 45, 80), b=128, dtype=1), B.OP_ATTN) == lists
    # Gram matrix: one D x D fp32 partial per 2048 tokens (bf16 only)
    assert B.workspace_bytes(p, B.OP_GRAM) == al(4 * 40 * 37 * 128 * 128)
    assert B.workspace_bytes(prob(heads=40, grid=(21, 45, 80), b=128, dtype=1), B.OP_GRAM) == 0
    # k-means: 2 G c split (2 x fp16) and fp32, b, block maxima, chunk histograms, ranks, offsets,
    # fp64 run sums of the mean segments (two per 256 sorted positions), then per chunk of 32
    # centroids their b and unscale factors together (what the assignment loads with the chunk)
    nch = -(-75600 // 256)
    assert B.workspace_bytes(p, B.OP_KMEANS) == (2 * al(2 * 40 * nbp * 128) + al(4 * 40 * nbp * 128)
                                                 + al(4 * 40 * nbp) + al(4 * 40 * 591) + al(4 * 40 * nch * 591)
                                                 + al(4 * 40 * 75600) + al(4 * 40 * 591)
                                                 + al(8 * 40 * nch * 2 * 128) + al(8 * 40 * nbp))
    # cluster attention: k and v in the padded cluster layout, starts, sub-tile tables
    npad = -(-(75600 + 31 * 591) // 32) * 32
    rows = 40 * 591
    assert B.workspace_bytes(p, B.OP_CLUSTER_ATTN) == (2 * al(2 * 40 * npad * 128) + 4 * al(4 * rows)
                                                       + al(4 * rows * (npad // 32)) + al(4 * 8 * 10 * 296))
    # query-pooled scorer: pooled q and k, then block maxima
    assert B.workspace_bytes(p, B.OP_POOLED) == 2 * al(4 * 40 * 591 * 128) + al(4 * 40 * 591)
    assert B.workspace_bytes(prob(d=96), B.OP_SCORE) == 0          # invalid problem -> 0


@pytest.mark.parametrize("kw,code", [
    (dict(grid=(4, 8, 8), heads=0), SHAPE),
    (dict(d=96), SHAPE),
    (dict(b=32), SHAPE),
    (dict(grid=(64, 100, 90), b=64), SHAPE),                # 9000 blocks > 4096
    (dict(dtype=5), DTYPE),
    (dict(scale=float("inf")), ARG),
])
def test_problem_validation(lib, kw, code):
    p = prob(**kw)
    q, k, s, ws = Buf(), Buf(), Buf(), Buf(1 << 20)
    st = lib.rsa_score_blocks(ctypes.byref(p), q.ptr, k.ptr, None, s.ptr, ws.ptr, 1 << 20, None)
    assert st == code
    assert q.untouched() and k.untouched() and s.untouched() and ws.untouched()


def test_tokens_must_match_grid(lib):
    p = prob()
    p.tokens += 1
    b = Buf()
    assert lib.rsa_block_sparse_attn(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, b.ptr,
                                     None, None, 0, None) == SHAPE
    assert b.untouched()


def test_null_problem_and_pointers(lib):
    b = Buf()
    assert lib.rsa_score_blocks(None, b.ptr, b.ptr, None, b.ptr, b.ptr, 1 << 30, None) == NULL
    p = prob()
    assert lib.rsa_score_blocks(ctypes.byref(p), None, b.ptr, None, b.ptr, b.ptr, 1 << 30, None) == NULL
    assert lib.rsa_select_topp(ctypes.byref(p), b.ptr, None, 0, None, b.ptr, b.ptr, b.ptr, None,
                               None, 0, None) == NULL
    assert lib.rsa_mask_drift(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, 0.05, 1, None, b.ptr,
                              b.ptr, 1 << 30, None) == NULL
    assert lib.rsa_block_sparse_attn(ctypes.byref(p), b.ptr, b.ptr, None, b.ptr, b.ptr, b.ptr, None,
                                     None, 0, None) == NULL
    assert lib.rsa_dense_block_mass(ctypes.byref(p), b.ptr, b.ptr, None, None) == NULL
    assert lib.rsa_dense_block_mass(None, b.ptr, b.ptr, b.ptr, None) == NULL
    assert lib.rsa_score_blocks_pooled(ctypes.byref(p), b.ptr, None, b.ptr, b.ptr, 1 << 30, None) == NULL
    # the omitted-block attention needs its lse (the cache's weight)
    assert lib.rsa_attn_omitted(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, None, b.ptr, None,
                                b.ptr, 1 << 30, None) == NULL
    assert lib.rsa_attn_merge(ctypes.byref(p), b.ptr, b.ptr, b.ptr, None, None) == NULL
    assert lib.rsa_attn_merge(None, b.ptr, b.ptr, b.ptr, b.ptr, None) == NULL
    # the corrected attention needs the cached part and writes an lse
    assert lib.rsa_block_sparse_attn_corrected(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, None, b.ptr,
                                               b.ptr, b.ptr, b.ptr, 1 << 30, None) == NULL
    assert lib.rsa_block_sparse_attn_corrected(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, b.ptr,
                                               b.ptr, None, b.ptr, 1 << 30, None) == NULL
    assert lib.rsa_query_gram(ctypes.byref(p), None, b.ptr, b.ptr, 1 << 30, None) == NULL
    assert lib.rsa_score_clusters(ctypes.byref(p), b.ptr, b.ptr, None, b.ptr, b.ptr, 1 << 30, None) == NULL
    assert lib.rsa_cluster_attn(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, None, b.ptr, b.ptr, b.ptr, b.ptr,
                                b.ptr, 1 << 30, None) == NULL
    assert lib.rsa_kmeans(ctypes.byref(p), b.ptr, b.ptr, 3, 1, b.ptr, b.ptr, None, b.ptr, b.ptr, 1 << 30,
                          None) == NULL
    assert b.untouched()


def test_alignment(lib):
    p = prob()
    b = Buf()
    mis = ctypes.c_void_p(b.view.ctypes.data + 8)
    assert lib.rsa_block_sparse_attn(ctypes.byref(p), mis, b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, None,
                                     b.ptr, 1 << 30, None) == ALIGN
    assert lib.rsa_score_blocks(ctypes.byref(p), b.ptr, b.ptr, None, mis, b.ptr, 1 << 30, None) == ALIGN
    assert lib.rsa_dense_block_mass(ctypes.byref(p), b.ptr, mis, b.ptr, None) == ALIGN
    assert lib.rsa_score_blocks_pooled(ctypes.byref(p), b.ptr, b.ptr, mis, b.ptr, 1 << 30, None) == ALIGN
    assert lib.rsa_attn_omitted(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, None, mis, b.ptr,
                                b.ptr, 1 << 30, None) == ALIGN
    assert lib.rsa_attn_merge(ctypes.byref(p), b.ptr, b.ptr, mis, b.ptr, None) == ALIGN
    assert lib.rsa_block_sparse_attn_corrected(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, mis, b.ptr,
                                               b.ptr, b.ptr, b.ptr, 1 << 30, None) == ALIGN
    assert b.untouched()


def test_workspace_checks(lib):
    p = prob()
    b = Buf()
    need = B.workspace_bytes(p, B.OP_SCORE)
    assert lib.rsa_score_blocks(ctypes.byref(p), b.ptr, b.ptr, None, b.ptr, None, need, None) == WS
    assert lib.rsa_score_blocks(ctypes.byref(p), b.ptr, b.ptr, None, b.ptr, b.ptr, need - 1, None) == WS
    mis = ctypes.c_void_p(b.view.ctypes.data + 16)
    assert lib.rsa_score_blocks(ctypes.byref(p), b.ptr, b.ptr, None, b.ptr, mis, need, None) == WS
    aneed = B.workspace_bytes(p, B.OP_ATTN)
    assert lib.rsa_block_sparse_attn(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, None,
                                     b.ptr, aneed - 1, None) == WS
    assert lib.rsa_attn_omitted(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, b.ptr, None, b.ptr, b.ptr,
                                b.ptr, aneed - 1, None) == WS
    pneed = B.workspace_bytes(p, B.OP_POOLED)
    assert lib.rsa_score_blocks_pooled(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, pneed - 1, None) == WS
    assert lib.rsa_score_blocks_pooled(ctypes.byref(p), b.ptr, b.ptr, b.ptr, None, pneed, None) == WS
    dneed = B.workspace_bytes(p, B.OP_DRIFT)
    assert lib.rsa_mask_drift(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, 0.05, 1, b.ptr, b.ptr,
                              b.ptr, dneed - 8, None) == WS
    assert b.untouched()


def test_scalar_arguments(lib):
    p = prob()
    b = Buf()
    assert lib.rsa_mask_drift(ctypes.byref(p), b.ptr, b.ptr, b.ptr, b.ptr, float("nan"), 1, b.ptr,
                              b.ptr, b.ptr, 1 << 30, None) == ARG
    assert lib.rsa_select_topp(ctypes.byref(p), b.ptr, b.ptr, -1, None, b.ptr, b.ptr, b.ptr, None,
                               None, 0, None) == ARG
    for iters in (0, -2, 1001):                             # k-means runs 1..1000 iterations
        assert lib.rsa_kmeans(ctypes.byref(p), b.ptr, b.ptr, iters, 1, b.ptr, b.ptr, b.ptr, b.ptr, b.ptr,
                              1 << 30, None) == ARG
    assert b.untouched()


def test_binding_raises_named_error():
    p = prob(d=96)
    with pytest.raises(R.RsaError) as e:
        B._check(R.lib().rsa_score_blocks(ctypes.byref(p), None, None, None, None, None, 0, None),
                 "rsa_score_blocks")
    assert e.value.name == "RSA_ERR_SHAPE" and e.value.status == SHAPE
