"""MI355X-native block-sparse attention scoring (gfx950 HIP kernels behind a C ABI).

The hot path is four library calls (include/rsa.h): PARK block scoring,
top-p selection, the per-head drift check of Temporal Mask Reuse and
block-sparse flash attention.  Two more calls measure block retrieval
accuracy (dense block mass, query-pooled comparison scores) and three carry
RECAP's cached correction (attention over the omitted blocks, the join of two
attentions over disjoint key sets, and sparse attention joined with the cached
part in one pass); four more build PARK's query-aware key
clusters and use them as key blocks (Gram matrix of the queries, k-means,
cluster scores, cluster attention).  This package is only their ctypes
binding plus the host loops that reuse cached masks across denoising steps
and run the clustered path.
"""
from .binding import (Problem, RsaError, RsaLibraryMissing, attn_merge, attn_omitted,
                      block_sparse_attn, block_sparse_attn_corrected, cluster_attn, declared_functions, kmeans, query_gram, score_clusters,
                      dense_block_mass, lib, make_problem, mask_drift, score_blocks, score_blocks_noalloc,
                      score_blocks_pooled, select_topp, workspace_bytes, OP_ATTN, OP_DRIFT,
                      OP_CLUSTER_ATTN, OP_GRAM, OP_KMEANS, OP_POOLED, OP_SCORE, OP_SELECT, RSA_BF16, RSA_FP32, LIB_PATH)
from .cache import MaskCache

__all__ = [
    "Problem", "RsaError", "RsaLibraryMissing", "attn_merge", "attn_omitted", "block_sparse_attn",
    "block_sparse_attn_corrected",
    "cluster_attn", "declared_functions", "kmeans", "query_gram", "score_clusters", "OP_CLUSTER_ATTN",
    "OP_GRAM", "OP_KMEANS",
    "dense_block_mass", "lib", "make_problem", "mask_drift", "score_blocks", "score_blocks_noalloc",
    "score_blocks_pooled",
    "select_topp", "workspace_bytes", "MaskCache", "OP_ATTN", "OP_DRIFT", "OP_POOLED", "OP_SCORE",
    "OP_SELECT", "RSA_BF16", "RSA_FP32", "LIB_PATH",
]
