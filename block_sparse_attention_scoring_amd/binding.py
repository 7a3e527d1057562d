"""Thin ctypes binding of librsa (include/rsa.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels.  torch supplies
device memory and the current stream; no torch operator touches the data
here (outputs are only allocated with ``torch.empty``/``torch.zeros``).
If the library has not been built the first call raises ``RsaLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "librsa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "rsa.h")

RSA_BF16, RSA_FP32 = 0, 1
OP_SCORE, OP_SELECT, OP_DRIFT, OP_ATTN, OP_POOLED, OP_GRAM, OP_KMEANS, OP_CLUSTER_ATTN = range(8)


class RsaLibraryMissing(RuntimeError):
    pass


class RsaError(RuntimeError):
    def __init__(self, status: int, name: str, call: str):
        super().__init__(f"{call} failed: {name} ({status})")
        self.status = status
        self.name = name


class Problem(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32),
        ("tokens", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("grid_f", ctypes.c_int32),
        ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]

    @property
    def nblocks(self) -> int:
        return -(-self.tokens // self.block)

    def __repr__(self):
        return ("Problem(heads=%d, tokens=%d, head_dim=%d, grid=(%d,%d,%d), block=%d, dtype=%d, scale=%g)"
                % (self.heads, self.tokens, self.head_dim, self.grid_f, self.grid_h, self.grid_w,
                   self.block, self.dtype, self.softmax_scale))


_P = ctypes.c_void_p
_lib = None


def _declare(lib):
    pp = ctypes.POINTER(Problem)
    sz, i32, f32 = ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    sigs = {
        "rsa_workspace_bytes": (sz, [pp, i32]),
        "rsa_status_str": (ctypes.c_char_p, [i32]),
        "rsa_version": (i32, []),
        "rsa_score_blocks": (i32, [pp, _P, _P, _P, _P, _P, sz, _P]),
        "rsa_select_topp": (i32, [pp, _P, _P, i32, _P, _P, _P, _P, _P, _P, sz, _P]),
        "rsa_mask_drift": (i32, [pp, _P, _P, _P, _P, f32, i32, _P, _P, _P, sz, _P]),
        "rsa_block_sparse_attn": (i32, [pp, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]),
        "rsa_dense_block_mass": (i32, [pp, _P, _P, _P, _P]),
        "rsa_score_blocks_pooled": (i32, [pp, _P, _P, _P, _P, sz, _P]),
        "rsa_attn_omitted": (i32, [pp, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]),
        "rsa_attn_merge": (i32, [pp, _P, _P, _P, _P, _P]),
        "rsa_block_sparse_attn_corrected": (i32, [pp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]),
        "rsa_query_gram": (i32, [pp, _P, _P, _P, sz, _P]),
        "rsa_kmeans": (i32, [pp, _P, _P, i32, i32, _P, _P, _P, _P, _P, sz, _P]),
        "rsa_score_clusters": (i32, [pp, _P, _P, _P, _P, _P, sz, _P]),
        "rsa_cluster_attn": (i32, [pp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, sz, _P]),
        "rsa_score_blocks_noalloc": (i32, [pp, _P, _P, _P, _P, _P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def lib():
    """The loaded librsa (raises RsaLibraryMissing when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RsaLibraryMissing(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/rsa.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b(rsa_\w+)\s*\(", text, re.M)))


def _check(status: int, call: str):
    if status != 0:
        raise RsaError(status, lib().rsa_status_str(status).decode(), call)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape, optional: bool = False):
    """Reject, before any library call, a tensor the C entry points would
    misread: they take bare device pointers to dense row-major arrays."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major); call .contiguous() first")


def _gpu(**tensors):
    """Every given tensor (None allowed) must live on the GPU; checked after
    the dtype/shape/layout checks of the same call."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")


def _io_dtype(p: "Problem") -> torch.dtype:
    return torch.bfloat16 if p.dtype == RSA_BF16 else torch.float32


def _need_qkv(p: "Problem", **tensors):
    dt, shp = _io_dtype(p), (p.heads, p.tokens, p.head_dim)
    for name, t in tensors.items():
        _need(t, name, dt, shp)


def _need_lists(p: "Problem", counts, block_idx):
    nb = p.nblocks
    _need(counts, "counts", torch.int32, (p.heads, nb))
    _need(block_idx, "block_idx", torch.int32, (p.heads, nb, nb))


def _need_workspace(ws: Optional[torch.Tensor]):
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return RSA_BF16
    if dt == torch.float32:
        return RSA_FP32
    raise TypeError(f"unsupported dtype {dt}: q/k/v must be bfloat16 or float32")


def make_problem(q: torch.Tensor, grid, block: int, softmax_scale: float = 0.0) -> Problem:
    """Descriptor for q/k/v of shape [heads, tokens, head_dim] on a (F, H, W) grid."""
    h, n, d = q.shape
    f, y, x = grid
    return Problem(h, n, d, f, y, x, block, _dtype_code(q.dtype), float(softmax_scale))


def workspace_bytes(p: Problem, op: int) -> int:
    return int(lib().rsa_workspace_bytes(ctypes.byref(p), op))


def _workspace(p: Problem, op: int, device, ws: Optional[torch.Tensor]):
    need = workspace_bytes(p, op)
    if need == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def score_blocks(q, k, p: Problem, head_active=None, out=None, workspace=None):
    """PARK block scores [heads, NB, NB] fp32 (rsa_score_blocks)."""
    _need_qkv(p, q=q, k=k)
    _need(head_active, "head_active", torch.uint8, (p.heads,), optional=True)
    _need(out, "out", torch.float32, (p.heads, p.nblocks, p.nblocks), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, k=k, head_active=head_active, out=out, workspace=workspace)
    nb = p.nblocks
    if out is None:
        out = torch.empty((p.heads, nb, nb), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(p, OP_SCORE, q.device, workspace)
    _check(lib().rsa_score_blocks(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(head_active), _ptr(out),
                                  _ptr(ws), wsb, _stream(q)), "rsa_score_blocks")
    return out


def score_blocks_noalloc(q, k, p: Problem, head_active=None, out=None):
    """PARK block scores with the library's static workspace (rsa_score_blocks_noalloc):
    no device allocation by the library; ``out`` may be given to allocate nothing at all."""
    _need_qkv(p, q=q, k=k)
    _need(head_active, "head_active", torch.uint8, (p.heads,), optional=True)
    _need(out, "out", torch.float32, (p.heads, p.nblocks, p.nblocks), optional=True)
    _gpu(q=q, k=k, head_active=head_active, out=out)
    nb = p.nblocks
    if out is None:
        out = torch.empty((p.heads, nb, nb), dtype=torch.float32, device=q.device)
    _check(lib().rsa_score_blocks_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(head_active), _ptr(out),
                                          _stream(q)), "rsa_score_blocks_noalloc")
    return out


def select_topp(scores, top_p, p: Problem, max_blocks: int = 0, head_active=None, mask=None,
                counts=None, block_idx=None, density=None, want_density: bool = True):
    """Top-p selection -> (mask u8, counts i32, block_idx i32, density fp32 or None)."""
    nbq = p.nblocks
    _need(scores, "scores", torch.float32, (p.heads, nbq, nbq))
    _need(top_p, "top_p", torch.float32, (p.heads,))
    _need(head_active, "head_active", torch.uint8, (p.heads,), optional=True)
    _need(mask, "mask", torch.uint8, (p.heads, nbq, nbq), optional=True)
    _need(counts, "counts", torch.int32, (p.heads, nbq), optional=True)
    _need(block_idx, "block_idx", torch.int32, (p.heads, nbq, nbq), optional=True)
    _need(density, "density", torch.float32, (p.heads,), optional=True)
    _gpu(scores=scores, top_p=top_p, head_active=head_active, mask=mask, counts=counts, block_idx=block_idx, density=density)
    nb = p.nblocks
    dev = scores.device
    if mask is None:
        mask = torch.zeros((p.heads, nb, nb), dtype=torch.uint8, device=dev)
    if counts is None:
        counts = torch.zeros((p.heads, nb), dtype=torch.int32, device=dev)
    if block_idx is None:
        block_idx = torch.zeros((p.heads, nb, nb), dtype=torch.int32, device=dev)
    if density is None and want_density:
        density = torch.zeros((p.heads,), dtype=torch.float32, device=dev)
    _check(lib().rsa_select_topp(ctypes.byref(p), _ptr(scores), _ptr(top_p), int(max_blocks),
                                 _ptr(head_active), _ptr(mask), _ptr(counts), _ptr(block_idx),
                                 _ptr(density), None, 0, _stream(scores)), "rsa_select_topp")
    return mask, counts, block_idx, density


def mask_drift(q, k, q_ref, k_ref, p: Problem, threshold: float, update_ref: bool = True,
               drift=None, refresh=None, workspace=None):
    """Per-head drift and refresh flags -> (drift fp32 [H], refresh u8 [H])."""
    _need_qkv(p, q=q, k=k, q_ref=q_ref, k_ref=k_ref)
    _need(drift, "drift", torch.float32, (p.heads,), optional=True)
    _need(refresh, "refresh", torch.uint8, (p.heads,), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, k=k, q_ref=q_ref, k_ref=k_ref, drift=drift, refresh=refresh, workspace=workspace)
    if drift is None:
        drift = torch.empty((p.heads,), dtype=torch.float32, device=q.device)
    if refresh is None:
        refresh = torch.empty((p.heads,), dtype=torch.uint8, device=q.device)
    ws, wsb = _workspace(p, OP_DRIFT, q.device, workspace)
    _check(lib().rsa_mask_drift(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(q_ref), _ptr(k_ref),
                                float(threshold), int(bool(update_ref)), _ptr(drift), _ptr(refresh),
                                _ptr(ws), wsb, _stream(q)), "rsa_mask_drift")
    return drift, refresh


def block_sparse_attn(q, k, v, counts, block_idx, p: Problem, out=None, lse=None,
                      want_lse: bool = True, workspace=None):
    """Attention over the listed key blocks -> (out like q, lse fp32 [H, N] or None)."""
    _need_qkv(p, q=q, k=k, v=v)
    _need_lists(p, counts, block_idx)
    _need(out, "out", _io_dtype(p), (p.heads, p.tokens, p.head_dim), optional=True)
    _need(lse, "lse", torch.float32, (p.heads, p.tokens), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, k=k, v=v, counts=counts, block_idx=block_idx, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((p.heads, p.tokens), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(p, OP_ATTN, q.device, workspace)
    _check(lib().rsa_block_sparse_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(counts),
                                       _ptr(block_idx), _ptr(out), _ptr(lse), _ptr(ws), wsb,
                                       _stream(q)), "rsa_block_sparse_attn")
    return out, lse


def dense_block_mass(q, k, p: Problem, out=None):
    """Dense attention mass of each query block per key block [heads, NB, NB] fp32."""
    _need_qkv(p, q=q, k=k)
    _need(out, "out", torch.float32, (p.heads, p.nblocks, p.nblocks), optional=True)
    _gpu(q=q, k=k, out=out)
    nb = p.nblocks
    if out is None:
        out = torch.empty((p.heads, nb, nb), dtype=torch.float32, device=q.device)
    _check(lib().rsa_dense_block_mass(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(out), _stream(q)),
           "rsa_dense_block_mass")
    return out


def score_blocks_pooled(q, k, p: Problem, out=None, workspace=None):
    """Query-pooled comparison scores [heads, NB, NB] fp32 (rsa_score_blocks_pooled)."""
    _need_qkv(p, q=q, k=k)
    _need(out, "out", torch.float32, (p.heads, p.nblocks, p.nblocks), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, k=k, out=out, workspace=workspace)
    nb = p.nblocks
    if out is None:
        out = torch.empty((p.heads, nb, nb), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(p, OP_POOLED, q.device, workspace)
    _check(lib().rsa_score_blocks_pooled(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(out), _ptr(ws), wsb,
                                         _stream(q)), "rsa_score_blocks_pooled")
    return out


def attn_omitted(q, k, v, counts, block_idx, p: Problem, head_active=None, out=None, lse=None,
                 workspace=None):
    """Attention over the key blocks each row's list leaves out -> (out like q, lse fp32 [H, N]).

    Heads with head_active[h] == 0 keep what ``out``/``lse`` held (pass the
    cache's buffers to refresh only some heads)."""
    _need_qkv(p, q=q, k=k, v=v)
    _need_lists(p, counts, block_idx)
    _need(head_active, "head_active", torch.uint8, (p.heads,), optional=True)
    _need(out, "out", _io_dtype(p), (p.heads, p.tokens, p.head_dim), optional=True)
    _need(lse, "lse", torch.float32, (p.heads, p.tokens), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, k=k, v=v, counts=counts, block_idx=block_idx, head_active=head_active, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((p.heads, p.tokens), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(p, OP_ATTN, q.device, workspace)
    _check(lib().rsa_attn_omitted(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(counts),
                                  _ptr(block_idx), _ptr(head_active), _ptr(out), _ptr(lse), _ptr(ws),
                                  wsb, _stream(q)), "rsa_attn_omitted")
    return out, lse


def attn_merge(out, lse, part_out, part_lse, p: Problem):
    """In place: (out, lse) <- attention over the union of two disjoint key sets."""
    _need_qkv(p, out=out, part_out=part_out)
    _need(lse, "lse", torch.float32, (p.heads, p.tokens))
    _need(part_lse, "part_lse", torch.float32, (p.heads, p.tokens))
    _gpu(out=out, part_out=part_out, lse=lse, part_lse=part_lse)
    _check(lib().rsa_attn_merge(ctypes.byref(p), _ptr(out), _ptr(lse), _ptr(part_out), _ptr(part_lse),
                                _stream(out)), "rsa_attn_merge")
    return out, lse


def block_sparse_attn_corrected(q, k, v, counts, block_idx, part_out, part_lse, p: Problem, out=None, lse=None,
                                workspace=None):
    """Sparse attention over the lists joined with a cached complementary part
    in one pass -> (out like q, lse fp32 [H, N]) (rsa_block_sparse_attn_corrected).
    ``out``/``lse`` may be ``part_out``/``part_lse`` (in place)."""
    _need_qkv(p, q=q, k=k, v=v, part_out=part_out)
    _need_lists(p, counts, block_idx)
    _need(part_lse, "part_lse", torch.float32, (p.heads, p.tokens))
    _need(out, "out", _io_dtype(p), (p.heads, p.tokens, p.head_dim), optional=True)
    _need(lse, "lse", torch.float32, (p.heads, p.tokens), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, k=k, v=v, part_out=part_out, counts=counts, block_idx=block_idx, part_lse=part_lse, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((p.heads, p.tokens), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(p, OP_ATTN, q.device, workspace)
    _check(lib().rsa_block_sparse_attn_corrected(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(counts),
                                                 _ptr(block_idx), _ptr(part_out), _ptr(part_lse), _ptr(out),
                                                 _ptr(lse), _ptr(ws), wsb, _stream(q)),
           "rsa_block_sparse_attn_corrected")
    return out, lse


def query_gram(q, p: Problem, out=None, workspace=None):
    """Gram matrix of the current queries, [heads, head_dim, head_dim] fp32 (rsa_query_gram)."""
    _need_qkv(p, q=q)
    _need(out, "out", torch.float32, (p.heads, p.head_dim, p.head_dim), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, out=out, workspace=workspace)
    if out is None:
        out = torch.empty((p.heads, p.head_dim, p.head_dim), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(p, OP_GRAM, q.device, workspace)
    _check(lib().rsa_query_gram(ctypes.byref(p), _ptr(q), _ptr(out), _ptr(ws), wsb, _stream(q)), "rsa_query_gram")
    return out


def kmeans(k, gram, p: Problem, iters: int, init: bool = True, centroids=None, labels=None, sizes=None,
           order=None, workspace=None):
    """Lloyd k-means of the keys in the metric of ``gram`` (rsa_kmeans)
    -> (centroids fp32 [H, NB, D], labels i32 [H, N], sizes i32 [H, NB], order i32 [H, N])."""
    _need_qkv(p, k=k)
    _need(gram, "gram", torch.float32, (p.heads, p.head_dim, p.head_dim))
    _need(centroids, "centroids", torch.float32, (p.heads, p.nblocks, p.head_dim), optional=True)
    _need(labels, "labels", torch.int32, (p.heads, p.tokens), optional=True)
    _need(sizes, "sizes", torch.int32, (p.heads, p.nblocks), optional=True)
    _need(order, "order", torch.int32, (p.heads, p.tokens), optional=True)
    _need_workspace(workspace)
    _gpu(k=k, gram=gram, centroids=centroids, labels=labels, sizes=sizes, order=order, workspace=workspace)
    nb, dev = p.nblocks, k.device
    if centroids is None:
        if not init:
            raise ValueError("kmeans without init needs starting centroids")
        centroids = torch.empty((p.heads, nb, p.head_dim), dtype=torch.float32, device=dev)
    if labels is None:
        labels = torch.empty((p.heads, p.tokens), dtype=torch.int32, device=dev)
    if sizes is None:
        sizes = torch.empty((p.heads, nb), dtype=torch.int32, device=dev)
    if order is None:
        order = torch.empty((p.heads, p.tokens), dtype=torch.int32, device=dev)
    ws, wsb = _workspace(p, OP_KMEANS, dev, workspace)
    _check(lib().rsa_kmeans(ctypes.byref(p), _ptr(k), _ptr(gram), int(iters), int(bool(init)), _ptr(centroids),
                            _ptr(labels), _ptr(sizes), _ptr(order), _ptr(ws), wsb, _stream(k)), "rsa_kmeans")
    return centroids, labels, sizes, order


def score_clusters(q, centroids, sizes, p: Problem, out=None, workspace=None):
    """PARK scores with clusters as key blocks, [heads, NB, NB] fp32 (rsa_score_clusters)."""
    _need_qkv(p, q=q)
    _need(centroids, "centroids", torch.float32, (p.heads, p.nblocks, p.head_dim))
    _need(sizes, "sizes", torch.int32, (p.heads, p.nblocks))
    _need(out, "out", torch.float32, (p.heads, p.nblocks, p.nblocks), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, centroids=centroids, sizes=sizes, out=out, workspace=workspace)
    nb = p.nblocks
    if out is None:
        out = torch.empty((p.heads, nb, nb), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(p, OP_SCORE, q.device, workspace)
    _check(lib().rsa_score_clusters(ctypes.byref(p), _ptr(q), _ptr(centroids), _ptr(sizes), _ptr(out), _ptr(ws),
                                    wsb, _stream(q)), "rsa_score_clusters")
    return out


def cluster_attn(q, k, v, sizes, order, counts, block_idx, p: Problem, out=None, lse=None, want_lse: bool = True,
                 workspace=None):
    """Attention over the listed clusters' keys -> (out like q, lse fp32 [H, N] or None) (rsa_cluster_attn)."""
    _need_qkv(p, q=q, k=k, v=v)
    _need(sizes, "sizes", torch.int32, (p.heads, p.nblocks))
    _need(order, "order", torch.int32, (p.heads, p.tokens))
    _need_lists(p, counts, block_idx)
    _need(out, "out", _io_dtype(p), (p.heads, p.tokens, p.head_dim), optional=True)
    _need(lse, "lse", torch.float32, (p.heads, p.tokens), optional=True)
    _need_workspace(workspace)
    _gpu(q=q, k=k, v=v, sizes=sizes, order=order, counts=counts, block_idx=block_idx, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((p.heads, p.tokens), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(p, OP_CLUSTER_ATTN, q.device, workspace)
    _check(lib().rsa_cluster_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sizes), _ptr(order),
                                  _ptr(counts), _ptr(block_idx), _ptr(out), _ptr(lse), _ptr(ws), wsb, _stream(q)),
           "rsa_cluster_attn")
    return out, lse
