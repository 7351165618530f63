"""Oracle: ragged pack and zero-fill unpack (test infrastructure only).

Pack ([dasc] §4.1 and Appendix B "Ragged (Scheme 2)"; [dasc-pp] Appendix B.2
"Insertion and reuse"): for every retained unit of every layer, copy it from
a dense checkpoint into a pool slot at layer offset o_l plus its rank among
the layer's retained units; then copy the checkpoint's (uncompressed) conv
state after the temporal payload ([dasc-pp] §4.4: the compressed pool stores
retained recurrent units and uncompressed convolution states).

Unpack with zero-fill, dasc-nr ([dasc] §4.2): restore the retained units
exactly, leave every omitted (local) unit at zero, restore the conv state.

Everything is a raw copy of bit patterns (uint32 for fp32 state, uint8 for
conv bytes), so -0.0, NaN payloads and denormals survive untouched and the
comparison with any other implementation is bit-exact.  Zero means the
all-zero bit pattern, +0.0.

Array layouts: a dense checkpoint is one row of a uint8 array
[n, plan.dense_bytes] holding, per layer, the state [H, d_v, d_k] fp32 with
k fastest, then every layer's conv bytes; a pool slot is one row of a uint8
array [slots, plan.slot_bytes] holding the retained units layer by layer,
then every layer's conv bytes.  A GDN unit is a whole head [d_v, d_k]; a KDA
unit (h, k) is the column S[h, :, k], stored as d_v contiguous floats.
"""
from __future__ import annotations

import numpy as np

from .plan import GDN, OraclePlan


def _state_words(row: np.ndarray, plan: OraclePlan, li: int) -> np.ndarray:
    """View of layer li's state in one dense checkpoint row as uint32
    [H, d_v, d_k]."""
    lay = plan.layers[li]
    a = plan.temporal_off[li]
    return row[a:a + lay.state_bytes].view(np.uint32).reshape(
        lay.n_heads, lay.d_v, lay.d_k)


def _pool_units(slot: np.ndarray, plan: OraclePlan, li: int) -> np.ndarray:
    """View of layer li's retained units in one pool slot row as uint32
    [r_l, unit words]."""
    lay = plan.layers[li]
    a = plan.pool_off[li]
    return slot[a:a + lay.r * lay.unit_bytes].view(np.uint32).reshape(
        lay.r, lay.unit_bytes // 4)


def pack(plan: OraclePlan, dense: np.ndarray, src_idx, pool: np.ndarray,
         dst_slot) -> None:
    """pool[dst_slot[i]] <- retained units and conv of dense[src_idx[i]]."""
    for s, d in zip(np.asarray(src_idx), np.asarray(dst_slot)):
        src = dense[int(s)]
        dst = pool[int(d)]
        for li, lay in enumerate(plan.layers):
            S = _state_words(src, plan, li)
            P = _pool_units(dst, plan, li)
            for j, u in enumerate(lay.retained_idx):
                if lay.kind == GDN:
                    P[j] = S[u].reshape(-1)          # whole head u
                else:
                    h, k = divmod(int(u), lay.d_k)
                    P[j] = S[h, :, k]                 # column S[h, :, k]
            a, b = plan.conv_off[li], plan.pool_conv_off[li]
            dst[b:b + lay.conv_bytes] = src[a:a + lay.conv_bytes]


def unpack_zero_fill(plan: OraclePlan, pool: np.ndarray, src_slot,
                     dense: np.ndarray, dst_idx) -> None:
    """dense[dst_idx[i]] <- retained units of pool[src_slot[i]], +0.0 in
    every local unit, and the stored conv bytes."""
    for s, d in zip(np.asarray(src_slot), np.asarray(dst_idx)):
        src = pool[int(s)]
        dst = dense[int(d)]
        for li, lay in enumerate(plan.layers):
            S = _state_words(dst, plan, li)
            P = _pool_units(src, plan, li)
            S[...] = 0                                # dasc-nr: locals stay zero
            for j, u in enumerate(lay.retained_idx):
                if lay.kind == GDN:
                    S[u] = P[j].reshape(lay.d_v, lay.d_k)
                else:
                    h, k = divmod(int(u), lay.d_k)
                    S[h, :, k] = P[j]
            a, b = plan.conv_off[li], plan.pool_conv_off[li]
            dst[a:a + lay.conv_bytes] = src[b:b + lay.conv_bytes]
