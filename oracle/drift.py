"""Per-head query-key drift and the refresh rule, fp64 (oracle; test infrastructure only).

HEART, Abstract (Temporal Mask Reuse): a head's cached mask stays in use
until a cheap per-head measure of how far its queries and keys have moved
rises above a threshold tau; then the mask is recomputed.  HASTE, Abstract:
the same kind of measure decides when mask prediction can be skipped.

Reading (the pages give no formula): the relative Frobenius change of the
head's stacked queries and keys since the snapshot taken when its mask was
last computed,

    d_h = sqrt(|Q_h - Qs_h|^2 + |K_h - Ks_h|^2) / sqrt(|Qs_h|^2 + |Ks_h|^2),

and "exceeds" is strict: refresh iff ``d_h > tau``.  A zero snapshot gives
``d_h = 0`` when nothing changed and ``+inf`` otherwise.
"""
import numpy as np


def drift(q: np.ndarray, k: np.ndarray, q_ref: np.ndarray, k_ref: np.ndarray) -> np.ndarray:
    """``[H, N, D]`` arrays -> ``d [H]`` (fp64)."""
    h = q.shape[0]
    out = np.empty(h, np.float64)
    for a in range(h):
        dq = (q[a] - q_ref[a]).ravel()
        dk = (k[a] - k_ref[a]).ravel()
        rq = q_ref[a].ravel()
        rk = k_ref[a].ravel()
        num = np.dot(dq, dq) + np.dot(dk, dk)
        den = np.dot(rq, rq) + np.dot(rk, rk)
        if den > 0.0:
            out[a] = np.sqrt(num) / np.sqrt(den)
        else:
            out[a] = 0.0 if num == 0.0 else np.inf
    return out


def refresh_decision(d: np.ndarray, tau: float) -> np.ndarray:
    """Refresh flags (u8): drift strictly above the float32 threshold."""
    return (np.asarray(d, np.float64) > float(np.float32(tau))).astype(np.uint8)
