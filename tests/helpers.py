"""Test-side helpers shared by the GPU parity tests (comparison only; no
step of the method lives here)."""
from __future__ import annotations

import sys

import numpy as np


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def mask_words(plan) -> np.ndarray:
    """uint32 mask over one dense checkpoint built from the oracle plan:
    all-ones on retained units and on the conv bytes, zero on local units."""
    m = np.zeros(plan.dense_bytes // 4, dtype=np.uint32)
    for li, L in enumerate(plan.layers):
        base = plan.temporal_off[li] // 4
        n = L.n_heads * L.d_v * L.d_k
        if L.kind == 0:
            keep = np.broadcast_to(L.retained[:, None, None], (L.n_heads, L.d_v, L.d_k))
        else:
            keep = np.broadcast_to(L.retained.reshape(L.n_heads, 1, L.d_k), (L.n_heads, L.d_v, L.d_k))
        m[base:base + n] = np.where(keep.reshape(-1), 0xFFFFFFFF, 0).astype(np.uint32)
    m[plan.B_temp_dense // 4:] = 0xFFFFFFFF
    return m


def local_mask_of_head(plan, li: int, h: int) -> np.ndarray:
    """bool [d_v, d_k]: True where the refresh writes (local units)."""
    L = plan.layers[li]
    if L.kind == 0:
        return np.full((L.d_v, L.d_k), not L.retained[h])
    return np.broadcast_to(~L.retained.reshape(L.n_heads, L.d_k)[h][None, :], (L.d_v, L.d_k))


def head_state(dense_row: np.ndarray, plan, li: int, h: int) -> np.ndarray:
    """float32 [d_v, d_k] view of one head inside a dense checkpoint row."""
    L = plan.layers[li]
    a = plan.temporal_off[li] + h * L.d_v * L.d_k * 4
    return dense_row[a:a + L.d_v * L.d_k * 4].view(np.float32).reshape(L.d_v, L.d_k)


def refresh_error(gpu: np.ndarray, ref64: np.ndarray, local: np.ndarray) -> float:
    """max |gpu - ref| over the written (local) entries, over the Frobenius
    norm of the fp64 scratch state; 0 for an all-zero reference."""
    nrm = float(np.linalg.norm(ref64))
    if nrm == 0.0:
        return float(np.max(np.abs(gpu[local]))) if local.any() else 0.0
    if not local.any():
        return 0.0
    return float(np.max(np.abs(gpu[local].astype(np.float64) - ref64[local]))) / nrm
