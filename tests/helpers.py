"""Test-side helpers shared by the tests (comparison and input layouts only;
no step of the method lives here)."""
from __future__ import annotations

import sys

import numpy as np

import workloads as W


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


def block_pattern_layers():
    """d = 128 KDA heads whose 32-channel blocks are full, empty, sparse or
    retained at a single edge channel (A_log -4 is retained at W_max = 64,
    A_log 1 is not: H_s = ln(eps) / g is about 680 and 4.6 tokens)."""
    f = np.float32
    keep = np.zeros((4, 128), bool)
    keep[0, :32] = True
    keep[0, 64:96:2] = True
    keep[0, 127] = True
    keep[1, [0, 96]] = True
    keep[2, :] = True
    keep[2, [31, 32]] = False
    a = np.where(keep, -4.0, 1.0).reshape(-1).astype(f)
    z = np.zeros(512, f)
    return [W.Layer(W.KDA, 4, 128, 128, a, z, 64), W.Layer(W.KDA, 4, 128, 128, a[::-1].copy(), z, 0)]
