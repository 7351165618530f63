"""Oracle: INT8 checkpoint storage, Eq. 10 (test infrastructure only).

[dasc] Appendix E.1 "INT8 state checkpoint protocol", Eq. 10: only the cached
fp32 temporal state is quantized; the conv state stays bf16.  For the state
S [L, H, d_v, d_k] one scale per (l, h, k), shared over d_v:

    a_{l,h,k} = max_v |S_{l,h,v,k}|
    s_{l,h,k} = max(a_{l,h,k}, 1e-8) / 127
    q         = clip(round(S / s), -127, 127)      symmetric, no zero point

with the maximum, the division and the rounding in fp32; q is stored as int8
and s as fp32.  On a hit the checkpoint is dequantized once, S_hat = q s, in
fp32.  Composed with the ragged layout ([dasc] §4.1, Appendix B Scheme 2)
only the retained units are stored: a retained GDN head keeps its d_k
column scales, a retained KDA unit (h, k) is exactly one column and keeps
one scale.

Because the page fixes the precision (fp32), this oracle computes in numpy
float32, step by step as printed, and compares bit for bit.

Readings (the page is silent on them):
* "round" is round-half-to-even (numpy rint), the IEEE default.
* max(., 1e-8) and the column maximum ignore NaN: a NaN entry's magnitude
  counts as 0 (the maximum of the other magnitudes, all >= 0, is then
  unchanged; numpy's fmax.reduce was seen to miss the maximum when a
  signaling NaN shares its vector block); a quotient S / s that is NaN (a
  NaN or infinite state entry) quantizes to 0.
* INT8 pool slot layout: every retained unit's int8 payload, layer by layer
  in unit order (a GDN unit as [d_v][d_k] row-major, a KDA unit as its d_v
  column entries), padded to 16 bytes; then every retained unit's fp32
  scales in the same order (d_k per GDN unit, one per KDA unit), padded to
  16 bytes; then every layer's conv bytes.
"""
from __future__ import annotations

import math

import numpy as np

from .plan import GDN, OraclePlan

F32 = np.float32
SCALE_FLOOR = F32(1e-8)
QMAX = F32(127.0)


def align16(x: int) -> int:
    return (x + 15) // 16 * 16


class Int8Layout:
    """Byte offsets of the INT8 pool slot for one plan."""

    def __init__(self, plan: OraclePlan):
        self.q_off, self.s_off = [], []
        q = s = 0
        for lay in plan.layers:
            self.q_off.append(q)
            self.s_off.append(s)
            per_unit_q = lay.d_v * lay.d_k if lay.kind == GDN else lay.d_v
            per_unit_s = lay.d_k if lay.kind == GDN else 1
            q += lay.r * per_unit_q
            s += lay.r * per_unit_s * 4
        self.payload_bytes = q
        self.scale_bytes = s
        self.scale_base = align16(q)
        self.conv_base = self.scale_base + align16(s)
        self.B_conv = plan.B_conv
        self.slot_bytes = self.conv_base + plan.B_conv
        self.dense_bytes = plan.dense_bytes

    @property
    def C_ckpt(self) -> float:
        """Checkpoint capacity ratio against the dense mixed-precision
        checkpoint, the quantity the page's 8.11x measures; unbounded (inf)
        when nothing is stored, as for Eq. 6's ratio."""
        return math.inf if self.slot_bytes == 0 else self.dense_bytes / self.slot_bytes


def quantize_columns(X: np.ndarray):
    """Eq. 10 on a block X [d_v, m] of fp32 columns (one scale per column).
    Returns (q int8 [d_v, m], s float32 [m])."""
    X = np.asarray(X, dtype=F32)
    mag = np.abs(X)
    a = np.where(np.isnan(mag), F32(0), mag).max(axis=0)  # max_v |S|, NaN entries skipped
    s = np.maximum(a, SCALE_FLOOR) / QMAX              # fp32 division
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.rint(X / s[None, :])                    # fp32 quotient, half to even
    r = np.where(np.isnan(r), F32(0), r)
    q = np.clip(r, -QMAX, QMAX).astype(np.int8)
    return q, s.astype(F32)


def dequantize_columns(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """S_hat = q s in fp32 (0 * inf = NaN for a column whose maximum was
    infinite, as the product defines)."""
    with np.errstate(invalid="ignore"):
        return (np.asarray(q, dtype=np.int8).astype(F32) * np.asarray(s, dtype=F32)[None, :]).astype(F32)


def _state(row: np.ndarray, plan: OraclePlan, li: int) -> np.ndarray:
    lay = plan.layers[li]
    a = plan.temporal_off[li]
    return row[a:a + lay.state_bytes].view(F32).reshape(lay.n_heads, lay.d_v, lay.d_k)


def pack_int8(plan: OraclePlan, dense: np.ndarray, src_idx, pool: np.ndarray, dst_slot) -> None:
    """pool[dst_slot[i]] <- Eq. 10 of the retained units of dense[src_idx[i]]
    (int8 payload and fp32 scales) and its conv bytes."""
    lo = Int8Layout(plan)
    for si, di in zip(np.asarray(src_idx), np.asarray(dst_slot)):
        src, dst = dense[int(si)], pool[int(di)]
        for li, lay in enumerate(plan.layers):
            S = _state(src, plan, li)
            qo, so = lo.q_off[li], lo.scale_base + lo.s_off[li]
            for j, u in enumerate(lay.retained_idx):
                if lay.kind == GDN:
                    q, s = quantize_columns(S[u])                      # [d_v, d_k], d_k scales
                    nq = lay.d_v * lay.d_k
                    dst[qo + j * nq:qo + (j + 1) * nq] = q.reshape(-1).view(np.uint8)
                    dst[so + j * lay.d_k * 4:so + (j + 1) * lay.d_k * 4] = s.view(np.uint8)
                else:
                    h, k = divmod(int(u), lay.d_k)
                    q, s = quantize_columns(S[h][:, k:k + 1])          # one column, one scale
                    dst[qo + j * lay.d_v:qo + (j + 1) * lay.d_v] = q[:, 0].view(np.uint8)
                    dst[so + j * 4:so + (j + 1) * 4] = s.view(np.uint8)
        dst[lo.conv_base:lo.conv_base + plan.B_conv] = src[plan.B_temp_dense:plan.dense_bytes]


def unpack_int8_zero_fill(plan: OraclePlan, pool: np.ndarray, src_slot, dense: np.ndarray,
                          dst_idx) -> None:
    """dense[dst_idx[i]] <- S_hat = q s for the retained units of
    pool[src_slot[i]], +0.0 in every local unit, and the stored conv bytes
    (dasc-nr, [dasc] §4.2, on the INT8 checkpoint)."""
    lo = Int8Layout(plan)
    for si, di in zip(np.asarray(src_slot), np.asarray(dst_idx)):
        src, dst = pool[int(si)], dense[int(di)]
        for li, lay in enumerate(plan.layers):
            S = _state(dst, plan, li)
            S[...] = F32(0)
            qo, so = lo.q_off[li], lo.scale_base + lo.s_off[li]
            for j, u in enumerate(lay.retained_idx):
                if lay.kind == GDN:
                    nq = lay.d_v * lay.d_k
                    q = src[qo + j * nq:qo + (j + 1) * nq].view(np.int8).reshape(lay.d_v, lay.d_k)
                    s = src[so + j * lay.d_k * 4:so + (j + 1) * lay.d_k * 4].view(F32)
                    S[u] = dequantize_columns(q, s)
                else:
                    h, k = divmod(int(u), lay.d_k)
                    q = src[qo + j * lay.d_v:qo + (j + 1) * lay.d_v].view(np.int8)
                    s = src[so + j * 4:so + (j + 1) * 4].view(F32)
                    S[h][:, k] = dequantize_columns(q[:, None], s)[:, 0]
        dst[plan.B_temp_dense:plan.dense_bytes] = src[lo.conv_base:lo.conv_base + plan.B_conv]
