"""Seeded synthetic inputs shaped like the pages' video-DiT attention workloads.

This module is shared by the oracle-side tests, the GPU parity tests and the
benchmark.  It only *generates inputs*: it holds none of the method's
arithmetic (no pooling, no softmax, no selection, no attention, no drift).

The pages measure on Wan2.1 (480p / 720p) and HunyuanVideo (720p, 5 s)
generation (PARK abstract; HASTE abstract; RAPID abstract; RECAP abstract).
Those need trained weights and prompts, which are not available, so the
inputs here stand in for them with the same latent shapes: q/k/v laid out
``[heads, tokens, head_dim]`` with tokens in (frame, height, width) order.

Recipe (per config ``c``, head ``h``):

* smooth field ``F(f,y,x) = sum_{m<8} a_m cos(2 pi (u_m f/F + v_m y/Y + w_m x/X) + phi_m)``
  with ``a_m ~ N(0, I_D / 8)``, integer frequencies ``(u,v,w)`` drawn from
  ``{0,1,2}^3 \\ {0}`` and ``phi_m ~ U[0, 2 pi)``;
* ``q = alpha_h F_qk + 0.3 eps``, ``k = alpha_h F_qk + 0.3 eps'`` (one shared
  field, so attention is local in the field), ``v = F_v + 0.3 eps''``;
* per-head sharpness ``alpha_h = alpha * 2**u_h`` with ``u_h ~ U(-1/2, 1/2)``
  (heads differ, as HEART's abstract observes);
* fp32 generation, then a round-to-nearest-even cast to bf16 for the bf16
  configs; the fp32 config keeps the fp32 values.

Seeds come from ``numpy.random.SeedSequence([c, h, tensor_id, step])`` with
``tensor_id`` q=0, k=1, v=2, field parameters 10/11, head sharpness 20.
The trajectory config perturbs the fp32 masters of q and k once per step by
``0.02 * N(0, 1)`` (a random walk) and casts every step to bf16; with
``values=True`` the v master takes the same walk (for the cached correction,
whose omitted part ages as the values move).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Sequence

import numpy as np
import torch

# Generator sharpness constant.  Chosen as the smallest value of
# {0.5, 0.75, 1, 1.5, 2, 3} for which the oracle's mean density on the
# Wan2.1-14B-like 720p shape at top-p 0.9 falls inside [0.15, 0.30]; the
# calibration is re-checked by tests/test_workloads.py.
ALPHA = 2.0

NOISE_STD = 0.3
DRIFT_STD = 0.02
N_MODES = 8

TID_Q, TID_K, TID_V = 0, 1, 2
TID_FIELD_QK, TID_FIELD_V = 10, 11
TID_ALPHA = 20


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int                 # config number used in the seeds
    name: str
    heads: int
    grid: tuple              # (F, Y, X) latent grid
    head_dim: int
    block: int
    dtype: str               # "bf16" or "fp32"
    top_p: tuple             # per-head top-p pattern, repeated over heads
    steps: int = 1           # > 1 only for the mask-reuse trajectory
    drift_threshold: float = 0.05
    seed_cid: int | None = None   # base inputs come from this config's seeds

    @property
    def tokens(self) -> int:
        f, y, x = self.grid
        return f * y * x

    @property
    def nblocks(self) -> int:
        return -(-self.tokens // self.block)

    def top_p_array(self) -> np.ndarray:
        pat = self.top_p
        return np.array([pat[h % len(pat)] for h in range(self.heads)], dtype=np.float32)

    def scaled(self, heads=None, grid=None, name=None):
        """Same recipe at another size (for oracle-sized parity cases)."""
        return dataclasses.replace(
            self, heads=heads or self.heads, grid=grid or self.grid,
            name=name or f"{self.name}-scaled")


CONFIGS = {
    "tiny": Workload(1, "tiny", 1, (4, 8, 8), 64, 64, "fp32", (0.9,)),
    "wan13b_480p": Workload(2, "wan13b_480p", 12, (21, 30, 52), 128, 64, "bf16", (0.8, 0.9, 0.95)),
    "wan14b_720p": Workload(3, "wan14b_720p", 40, (21, 45, 80), 128, 128, "bf16", (0.9,)),
    "hunyuan_720p": Workload(4, "hunyuan_720p", 24, (33, 45, 80), 128, 128, "bf16", (0.9,)),
    "reuse_720p": Workload(5, "reuse_720p", 40, (21, 45, 80), 128, 128, "bf16", (0.9,),
                           steps=50, drift_threshold=0.05, seed_cid=3),
}
ORDER = ["tiny", "wan13b_480p", "wan14b_720p", "hunyuan_720p", "reuse_720p"]


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(x) for x in key])))


_FREQS = np.array([(u, v, w) for u in range(3) for v in range(3) for w in range(3)
                   if (u, v, w) != (0, 0, 0)], dtype=np.float64)


def smooth_field(cid: int, h: int, tid: int, grid, head_dim: int) -> np.ndarray:
    """Low-frequency 3-D field sampled at every token, fp32 ``[N, D]``."""
    rng = _rng(cid, h, tid, 0)
    F, Y, X = grid
    freqs = _FREQS[rng.integers(0, len(_FREQS), size=N_MODES)]          # [M, 3]
    phase = rng.uniform(0.0, 2.0 * math.pi, size=N_MODES)                # [M]
    amp = rng.standard_normal((N_MODES, head_dim)) / math.sqrt(N_MODES)  # [M, D]
    f = np.arange(F, dtype=np.float64)[:, None, None] / F
    y = np.arange(Y, dtype=np.float64)[None, :, None] / Y
    x = np.arange(X, dtype=np.float64)[None, None, :] / X
    cols = []
    for m in range(N_MODES):
        u, v, w = freqs[m]
        arg = 2.0 * math.pi * (u * f + v * y + w * x) + phase[m]
        cols.append(np.cos(arg).reshape(-1))
    basis = np.stack(cols, axis=1)                                      # [N, M]
    return (basis @ amp).astype(np.float32)


def head_alpha(cid: int, h: int, alpha: float = ALPHA) -> float:
    u = _rng(cid, h, TID_ALPHA, 0).uniform(-0.5, 0.5)
    return float(alpha * 2.0 ** u)


def noise(cid: int, h: int, tid: int, step: int, n: int, d: int) -> np.ndarray:
    return _rng(cid, h, tid, step).standard_normal((n, d), dtype=np.float32)


def _head_masters(wl: Workload, h: int, alpha: float):
    cid = wl.seed_cid if wl.seed_cid is not None else wl.cid
    n, d = wl.tokens, wl.head_dim
    a = np.float32(head_alpha(cid, h, alpha))
    fqk = smooth_field(cid, h, TID_FIELD_QK, wl.grid, d)
    fv = smooth_field(cid, h, TID_FIELD_V, wl.grid, d)
    q = a * fqk + np.float32(NOISE_STD) * noise(cid, h, TID_Q, 0, n, d)
    k = a * fqk + np.float32(NOISE_STD) * noise(cid, h, TID_K, 0, n, d)
    v = fv + np.float32(NOISE_STD) * noise(cid, h, TID_V, 0, n, d)
    return q, k, v


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: torch.Tensor          # [H, N, D] in the workload dtype (CPU)
    k: torch.Tensor
    v: torch.Tensor
    top_p: np.ndarray        # [H] float32
    q_master: np.ndarray | None = None   # fp32 masters, kept for trajectories
    k_master: np.ndarray | None = None
    v_master: np.ndarray | None = None


def make_inputs(wl: Workload, alpha: float = ALPHA, heads: Sequence[int] | None = None,
                keep_masters: bool = False) -> Inputs:
    """Generate q/k/v for every head (or the listed heads) of a workload."""
    hs = list(range(wl.heads)) if heads is None else list(heads)
    n, d = wl.tokens, wl.head_dim
    qm = np.empty((len(hs), n, d), np.float32)
    km = np.empty_like(qm)
    vm = np.empty_like(qm)

    def one(i):
        qm[i], km[i], vm[i] = _head_masters(wl, hs[i], alpha)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(len(hs))))
    p = wl.top_p_array()[hs]
    out = Inputs(wl, _cast(qm, wl.dtype), _cast(km, wl.dtype), _cast(vm, wl.dtype), p)
    if keep_masters:
        out.q_master, out.k_master, out.v_master = qm, km, vm
    return out


def drift_step(inp: Inputs, step: int, heads: Sequence[int] | None = None,
               values: bool = False) -> None:
    """Advance the q/k (and with ``values``, v) fp32 masters by one random-walk
    step and re-cast."""
    wl = inp.workload
    assert inp.q_master is not None, "make_inputs(..., keep_masters=True) first"
    hs = list(range(wl.heads)) if heads is None else list(heads)
    n, d = wl.tokens, wl.head_dim
    s = np.float32(DRIFT_STD)

    def one(i):
        h = hs[i]
        inp.q_master[i] += s * noise(wl.cid, h, TID_Q, step, n, d)
        inp.k_master[i] += s * noise(wl.cid, h, TID_K, step, n, d)
        if values:
            inp.v_master[i] += s * noise(wl.cid, h, TID_V, step, n, d)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(len(hs))))
    inp.q = _cast(inp.q_master, wl.dtype)
    inp.k = _cast(inp.k_master, wl.dtype)
    if values:
        inp.v = _cast(inp.v_master, wl.dtype)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a CPU tensor (bf16 and fp32 values upcast exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()
