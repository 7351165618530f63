"""MI355X-native state-checkpoint hot path of decay-aware state compression.

A thin Python binding over the C ABI in include/dasc.h (libdasc.so, built for
gfx950 by `python recurrent_state_cache_amd/_build.py`).  This module only
marshals arguments: every step of the plan runs in the library's host code
and every step of pack, unpack and refresh runs in its HIP kernels.  There is
no fallback: if the library is missing, importing this package fails.

PyTorch supplies device memory and streams only.  Tensors passed to the data
calls must live on the GPU; the library never sees a torch type.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
# torch first: its HIP runtime (SONAME libamdhip64.so.7) must be the one the
# library binds to, so that torch's streams and allocations are valid here.
# Loading the library first would bring in a second, separate runtime.
import torch  # noqa: F401

__all__ = ["Plan", "DascError", "ckpt_pack", "ckpt_unpack_zero_fill",
           "ckpt_refresh_suffix", "ckpt_refresh_suffix_windowed",
           "ckpt_refresh_suffix_alpha", "ckpt_refresh_suffix_alpha_windowed",
           "ckpt_refresh_suffix_recurrent", "ckpt_pack_int8",
           "ckpt_unpack_int8_zero_fill", "ckpt_pack_tp", "ckpt_unpack_tp_zero_fill",
           "ckpt_unpack_refresh",
           "GDN", "KDA", "STATUS_BAD_INDEX",
           "STATUS_BAD_TOKENS", "LIB_PATH", "lib"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdasc.so")

GDN = 0
KDA = 1
STATUS_BAD_INDEX = 1
STATUS_BAD_TOKENS = 2

_c_i32, _c_i64, _c_f64, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p


class _LayerDesc(ctypes.Structure):
    _fields_ = [("kind", _c_i32), ("n_heads", _c_i32), ("d_k", _c_i32), ("d_v", _c_i32),
                ("A_log", ctypes.POINTER(ctypes.c_float)),
                ("dt_bias", ctypes.POINTER(ctypes.c_float)), ("conv_bytes", _c_i64)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("n_layers", _c_i32), ("w_replay", _c_i32), ("n_units", _c_i64),
                ("n_retained", _c_i64), ("temporal_dense_bytes", _c_i64),
                ("temporal_rag_bytes", _c_i64), ("conv_bytes", _c_i64),
                ("dense_bytes", _c_i64), ("slot_bytes", _c_i64), ("r_max", _c_i64),
                ("r_bar", _c_f64), ("c_temp", _c_f64), ("c_ckpt", _c_f64),
                ("c_temp_pad", _c_f64), ("layout_gain", _c_f64),
                ("n_refresh_heads", _c_i64), ("device_bytes", _c_i64), ("k_row", _c_i64),
                ("v_row", _c_i64), ("gate_row", _c_i64), ("beta_row", _c_i64),
                ("int8_payload_bytes", _c_i64), ("int8_scale_bytes", _c_i64),
                ("int8_slot_bytes", _c_i64), ("c_ckpt_int8", _c_f64)]


class _LayerInfo(ctypes.Structure):
    _fields_ = [("kind", _c_i32), ("n_heads", _c_i32), ("d_k", _c_i32), ("d_v", _c_i32),
                ("n_units", _c_i64), ("n_retained", _c_i64), ("unit_offset", _c_i64),
                ("unit_bytes", _c_i64), ("dense_offset", _c_i64),
                ("conv_dense_offset", _c_i64), ("pool_offset", _c_i64),
                ("conv_pool_offset", _c_i64), ("conv_bytes", _c_i64), ("w_layer", _c_i32),
                ("n_refresh_heads", _c_i32), ("k_row_offset", _c_i64),
                ("v_row_offset", _c_i64), ("gate_row_offset", _c_i64),
                ("beta_row_offset", _c_i64), ("int8_pool_offset", _c_i64),
                ("int8_scale_offset", _c_i64)]


class _TpInfo(ctypes.Structure):
    _fields_ = [("tp", _c_i32), ("rank", _c_i32), ("one_store", _c_i32), ("reserved", _c_i32),
                ("unit_bytes", _c_i64), ("n_total", _c_i64), ("slot_units", _c_i64),
                ("m_remote", _c_i64), ("max_local", _c_i64), ("n_local", _c_i64),
                ("target", _c_i64), ("keep", _c_i64), ("send_units", _c_i64),
                ("recv_units", _c_i64), ("slot_bytes", _c_i64), ("send_bytes", _c_i64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python recurrent_state_cache_amd/_build.py`")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "dasc_plan_build": (_c_i32, [ctypes.POINTER(_LayerDesc), _c_i32, _c_f64, _c_f64, _c_i32,
                                     ctypes.POINTER(_c_p)]),
        "dasc_plan_build_tp": (_c_i32, [ctypes.POINTER(_LayerDesc), _c_i32, _c_f64, _c_f64,
                                        _c_i32, _c_i32, _c_i32, ctypes.POINTER(_c_p)]),
        "dasc_plan_tp_info": (_c_i32, [_c_p, ctypes.POINTER(_TpInfo)]),
        "dasc_plan_tp_splits": (_c_i32, [_c_p, _c_p, _c_p, _c_p]),
        "dasc_ckpt_pack_tp": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_i64,
                                       _c_p, _c_p, _c_i64, _c_i64, _c_p, _c_i32, _c_p]),
        "dasc_ckpt_unpack_tp_zero_fill": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p,
                                                   _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_i64,
                                                   _c_p, _c_i32, _c_p]),
        "dasc_plan_query": (_c_i32, [_c_p, ctypes.POINTER(_PlanInfo)]),
        "dasc_plan_layer": (_c_i32, [_c_p, _c_i32, ctypes.POINTER(_LayerInfo)]),
        "dasc_plan_units": (_c_i32, [_c_p, _c_i32, _c_p, _c_p, _c_p]),
        "dasc_plan_slots": (_c_i64, [_c_p, _c_i64, _c_i32]),
        "dasc_plan_upload": (_c_i32, [_c_p, _c_p, _c_i64, _c_p]),
        "dasc_plan_status": (_c_i32, [_c_p, ctypes.POINTER(ctypes.c_uint32), _c_i32, _c_p]),
        "dasc_plan_launches": (_c_i32, [_c_p, _c_i32, _c_i32, ctypes.POINTER(_c_i32),
                                        ctypes.POINTER(_c_i32)]),
        "dasc_plan_destroy": (_c_i32, [_c_p]),
        "dasc_ckpt_pack": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_i64, _c_p,
                                    _c_i32, _c_p]),
        "dasc_ckpt_unpack_zero_fill": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64,
                                                _c_i64, _c_p, _c_i32, _c_p]),
        "dasc_ckpt_refresh_suffix": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p,
                                              _c_i64, _c_i64, _c_p, _c_i32, _c_p]),
        "dasc_ckpt_refresh_suffix_windowed": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                                       _c_p, _c_i64, _c_i64, _c_p, _c_i32, _c_p]),
        "dasc_ckpt_refresh_suffix_recurrent": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                                        _c_p, _c_i64, _c_i64, _c_p, _c_i32, _c_p]),
        "dasc_ckpt_refresh_suffix_alpha": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                                    _c_p, _c_i64, _c_i64, _c_p, _c_i32, _c_p]),
        "dasc_ckpt_refresh_suffix_alpha_windowed": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                                             _c_i64, _c_p, _c_i64, _c_i64, _c_p,
                                                             _c_i32, _c_p]),
        "dasc_ckpt_unpack_refresh": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p,
                                              _c_p, _c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_p,
                                              _c_i32, _c_i32, _c_p]),
        "dasc_ckpt_pack_int8": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_i64,
                                         _c_p, _c_i32, _c_p]),
        "dasc_ckpt_unpack_int8_zero_fill": (_c_i32, [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p,
                                                     _c_i64, _c_i64, _c_p, _c_i32, _c_p]),
        "dasc_last_error": (ctypes.c_char_p, []),
        "dasc_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()


class DascError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = lib.dasc_last_error().decode()
        super().__init__(f"{where}: code {code}: {msg}")
        self.code = code


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise DascError(rc, where)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev_ptr(t, name: str, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _rows(t, name: str):
    """(pointer, row stride in bytes, rows) of a 2-D uint8-viewable buffer."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows, bytes per row]")
    row_bytes = t.stride(0) * t.element_size()
    if t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    import torch
    if not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    return ctypes.c_void_p(t.data_ptr()), row_bytes, t.shape[0]


class Plan:
    """The static selection plan (host object owned by the library).

    `layers`: objects with kind (GDN / KDA), n_heads, d_k, d_v, A_log and
    dt_bias (float32, one per unit) and conv_bytes.  With tp > 1 the plan is
    rank `rank`'s (its own heads) with the storage-balancing map of all tp
    ranks.
    """

    def __init__(self, layers, a_s: float = -0.3, eps: float = 1e-3, w_max: int = 16,
                 tp: int = 1, rank: int = 0):
        descs = (_LayerDesc * len(layers))()
        keep = []
        for d, L in zip(descs, layers):
            A = np.ascontiguousarray(np.asarray(L.A_log, dtype=np.float32).reshape(-1))
            D = np.ascontiguousarray(np.asarray(L.dt_bias, dtype=np.float32).reshape(-1))
            keep += [A, D]
            d.kind, d.n_heads, d.d_k, d.d_v = int(L.kind), int(L.n_heads), int(L.d_k), int(L.d_v)
            d.A_log = A.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
            d.dt_bias = D.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
            d.conv_bytes = int(L.conv_bytes)
        h = _c_p()
        if tp == 1 and rank == 0:
            _check(lib.dasc_plan_build(descs, len(layers), float(a_s), float(eps), int(w_max),
                                       ctypes.byref(h)), "plan_build")
        else:
            _check(lib.dasc_plan_build_tp(descs, len(layers), float(a_s), float(eps),
                                          int(w_max), int(tp), int(rank), ctypes.byref(h)),
                   "plan_build_tp")
        self._h = h
        self._table = None
        self.n_layers = len(layers)

    # -- host queries -------------------------------------------------------
    def info(self) -> dict:
        i = _PlanInfo()
        _check(lib.dasc_plan_query(self._h, ctypes.byref(i)), "plan_query")
        return {f: getattr(i, f) for f, _ in _PlanInfo._fields_}

    def tp_info(self) -> dict:
        i = _TpInfo()
        _check(lib.dasc_plan_tp_info(self._h, ctypes.byref(i)), "plan_tp_info")
        return {f: getattr(i, f) for f, _ in _TpInfo._fields_}

    def tp_splits(self):
        """(send_units [tp, tp], n_local [tp], target [tp]) int64 arrays."""
        tp = self.tp_info()["tp"]
        M = np.zeros((tp, tp), np.int64)
        n = np.zeros(tp, np.int64)
        t = np.zeros(tp, np.int64)
        _check(lib.dasc_plan_tp_splits(self._h, M.ctypes.data, n.ctypes.data, t.ctypes.data),
               "plan_tp_splits")
        return M, n, t

    def layer(self, l: int) -> dict:
        i = _LayerInfo()
        _check(lib.dasc_plan_layer(self._h, int(l), ctypes.byref(i)), "plan_layer")
        return {f: getattr(i, f) for f, _ in _LayerInfo._fields_}

    def units(self, l: int):
        """(retained uint8, horizon float64, window int32) arrays of layer l."""
        n = self.layer(l)["n_units"]
        r = np.zeros(n, np.uint8)
        H = np.zeros(n, np.float64)
        w = np.zeros(n, np.int32)
        _check(lib.dasc_plan_units(self._h, int(l), r.ctypes.data, H.ctypes.data, w.ctypes.data),
               "plan_units")
        return r, H, w

    def slots(self, budget_bytes: int, dense: bool = False) -> int:
        return int(lib.dasc_plan_slots(self._h, int(budget_bytes), 1 if dense else 0))

    # -- device tables --------------------------------------------------------
    def upload(self, device="cuda", stream=None):
        import torch
        nbytes = self.info()["device_bytes"]
        t = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-t.data_ptr()) % 256
        view = t[off:off + nbytes]
        _check(lib.dasc_plan_upload(self._h, ctypes.c_void_p(view.data_ptr()), nbytes,
                                    _stream_handle(stream)), "plan_upload")
        self._table = t
        return self

    def status(self, clear: bool = True, stream=None) -> int:
        s = ctypes.c_uint32(0)
        _check(lib.dasc_plan_status(self._h, ctypes.byref(s), 1 if clear else 0,
                                    _stream_handle(stream)), "plan_status")
        return int(s.value)

    MOVERS = {"pack": 0, "unpack": 1, "pack_int8": 2, "unpack_int8": 3, "pack_tp": 4,
              "unpack_tp": 5}

    def launches(self, mover: str, n: int) -> tuple:
        """(launches, pairs per launch) of a mover call over n pairs."""
        nl, per = _c_i32(0), _c_i32(0)
        _check(lib.dasc_plan_launches(self._h, self.MOVERS[mover], int(n), ctypes.byref(nl),
                                      ctypes.byref(per)), "plan_launches")
        return int(nl.value), int(per.value)

    def close(self):
        h = getattr(self, "_h", None)
        self._h = None
        if h and lib is not None:   # lib is None during interpreter shutdown
            lib.dasc_plan_destroy(h)

    def __del__(self):
        self.close()


def ckpt_pack(plan: Plan, dense, src_idx, pool, dst_slot, stream=None) -> None:
    """pool[dst_slot[i]] <- retained units + conv of dense[src_idx[i]].
    dense: [n_dense, >= dense_bytes] and pool: [n_slots, >= slot_bytes]
    uint8 CUDA tensors; src_idx, dst_slot: int32 CUDA tensors of equal length."""
    import torch
    dp, ds, dn = _rows(dense, "dense")
    pp, ps, pn = _rows(pool, "pool")
    n = src_idx.numel()
    if dst_slot.numel() != n:
        raise ValueError("src_idx and dst_slot differ in length")
    _check(lib.dasc_ckpt_pack(plan._h, dp, ds, dn, _dev_ptr(src_idx, "src_idx", torch.int32),
                              pp, ps, pn, _dev_ptr(dst_slot, "dst_slot", torch.int32), n,
                              _stream_handle(stream)), "ckpt_pack")


def ckpt_unpack_zero_fill(plan: Plan, pool, src_slot, dense, dst_idx, stream=None) -> None:
    """dense[dst_idx[i]] <- retained units of pool[src_slot[i]], +0.0 in local
    units, and the stored conv bytes."""
    import torch
    pp, ps, pn = _rows(pool, "pool")
    dp, ds, dn = _rows(dense, "dense")
    n = src_slot.numel()
    if dst_idx.numel() != n:
        raise ValueError("src_slot and dst_idx differ in length")
    _check(lib.dasc_ckpt_unpack_zero_fill(plan._h, pp, ps, pn,
                                          _dev_ptr(src_slot, "src_slot", torch.int32), dp, ds, dn,
                                          _dev_ptr(dst_idx, "dst_idx", torch.int32), n,
                                          _stream_handle(stream)), "ckpt_unpack_zero_fill")


def ckpt_pack_int8(plan: Plan, dense, src_idx, pool, dst_slot, stream=None) -> None:
    """INT8 pool slot pool[dst_slot[i]] <- Eq. 10 of the retained units of
    dense[src_idx[i]] (int8 payload, fp32 scales) and its raw conv bytes.
    pool: [n_slots, >= int8_slot_bytes] uint8 CUDA tensor."""
    import torch
    dp, ds, dn = _rows(dense, "dense")
    pp, ps, pn = _rows(pool, "pool")
    n = src_idx.numel()
    if dst_slot.numel() != n:
        raise ValueError("src_idx and dst_slot differ in length")
    _check(lib.dasc_ckpt_pack_int8(plan._h, dp, ds, dn, _dev_ptr(src_idx, "src_idx", torch.int32),
                                   pp, ps, pn, _dev_ptr(dst_slot, "dst_slot", torch.int32), n,
                                   _stream_handle(stream)), "ckpt_pack_int8")


def ckpt_unpack_int8_zero_fill(plan: Plan, pool, src_slot, dense, dst_idx, stream=None) -> None:
    """dense[dst_idx[i]] <- q s in the retained units of INT8 slot
    pool[src_slot[i]], +0.0 in local units, and the stored conv bytes."""
    import torch
    pp, ps, pn = _rows(pool, "pool")
    dp, ds, dn = _rows(dense, "dense")
    n = src_slot.numel()
    if dst_idx.numel() != n:
        raise ValueError("src_slot and dst_idx differ in length")
    _check(lib.dasc_ckpt_unpack_int8_zero_fill(plan._h, pp, ps, pn,
                                               _dev_ptr(src_slot, "src_slot", torch.int32), dp,
                                               ds, dn, _dev_ptr(dst_idx, "dst_idx", torch.int32),
                                               n, _stream_handle(stream)),
           "ckpt_unpack_int8_zero_fill")


def _alt_rows(plan, t, name):
    if t is None:
        if plan.tp_info()["send_units"] > 0:
            raise ValueError(f"{name} rows are required: this rank stores units elsewhere")
        return ctypes.c_void_p(0), 0, 0
    return _rows(t, name)


def ckpt_pack_tp(plan: Plan, dense, src_idx, pool, dst_slot, send, send_idx,
                 stream=None) -> None:
    """Store with TP storage balancing, this rank's part: kept units and
    conv into pool[dst_slot[i]], the rest into send[send_idx[i]]."""
    import torch
    dp, ds, dn = _rows(dense, "dense")
    pp, ps, pn = _rows(pool, "pool")
    sp, ss, sn = _alt_rows(plan, send, "send")
    n = src_idx.numel()
    if dst_slot.numel() != n or (send_idx is not None and send_idx.numel() != n):
        raise ValueError("index arrays must have the same length")
    sidx = _dev_ptr(send_idx, "send_idx", torch.int32) if send_idx is not None else None
    _check(lib.dasc_ckpt_pack_tp(plan._h, dp, ds, dn, _dev_ptr(src_idx, "src_idx", torch.int32),
                                 pp, ps, pn, _dev_ptr(dst_slot, "dst_slot", torch.int32),
                                 sp, ss, sn, sidx, n, _stream_handle(stream)), "ckpt_pack_tp")


def ckpt_unpack_tp_zero_fill(plan: Plan, pool, src_slot, recv, recv_idx, dense, dst_idx,
                             stream=None) -> None:
    """Load with TP storage balancing, this rank's part after the inverse
    exchange: kept units from pool[src_slot[i]], the rest from
    recv[recv_idx[i]], zero-fill, conv from the slot, into dense[dst_idx[i]]."""
    import torch
    dp, ds, dn = _rows(dense, "dense")
    pp, ps, pn = _rows(pool, "pool")
    rp, rs, rn = _alt_rows(plan, recv, "recv")
    n = src_slot.numel()
    if dst_idx.numel() != n or (recv_idx is not None and recv_idx.numel() != n):
        raise ValueError("index arrays must have the same length")
    ridx = _dev_ptr(recv_idx, "recv_idx", torch.int32) if recv_idx is not None else None
    _check(lib.dasc_ckpt_unpack_tp_zero_fill(plan._h, pp, ps, pn,
                                             _dev_ptr(src_slot, "src_slot", torch.int32),
                                             rp, rs, rn, ridx, dp, ds, dn,
                                             _dev_ptr(dst_idx, "dst_idx", torch.int32), n,
                                             _stream_handle(stream)),
           "ckpt_unpack_tp_zero_fill")


def _refresh(fn, name, plan, k, v, a, beta, tok_off, dense, dst_idx, stream, alpha=False):
    """Marshal a refresh call; `a` holds bf16 gate logits, or fp32 decays
    when alpha is True (same row width)."""
    import torch
    n = dst_idx.numel()
    if tok_off.numel() != n + 1:
        raise ValueError("tok_off must have n+1 entries")
    T = k.shape[0]
    info = plan.info()
    an = "alpha" if alpha else "a"
    for nm, t, w in (("k", k, info["k_row"]), ("v", v, info["v_row"]),
                     (an, a, info["gate_row"]), ("beta", beta, info["beta_row"])):
        if t.dim() != 2 or t.shape[0] != T or t.shape[1] != w:
            raise ValueError(f"{nm} must be [{T}, {w}], got {tuple(t.shape)}")
    dp, ds, dn = _rows(dense, "dense")
    _check(fn(plan._h, _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
              _dev_ptr(a, an, torch.float32 if alpha else torch.bfloat16),
              _dev_ptr(beta, "beta", torch.float32),
              _dev_ptr(tok_off, "tok_off", torch.int64), T, dp, ds, dn,
              _dev_ptr(dst_idx, "dst_idx", torch.int32), n, _stream_handle(stream)), name)


def ckpt_refresh_suffix_alpha(plan: Plan, k, v, alpha, beta, tok_off, dense, dst_idx,
                              stream=None) -> None:
    """Bounded-suffix refresh with the decays given directly (Eq. 1 as
    written): alpha is fp32 [T, gate row] (one per channel for KDA layers,
    one per head for GDN layers); other arguments as ckpt_refresh_suffix."""
    _refresh(lib.dasc_ckpt_refresh_suffix_alpha, "ckpt_refresh_suffix_alpha", plan, k, v,
             alpha, beta, tok_off, dense, dst_idx, stream, alpha=True)


def ckpt_refresh_suffix_alpha_windowed(plan: Plan, k, v, alpha, beta, tok_off, dense, dst_idx,
                                       stream=None) -> None:
    """ckpt_refresh_suffix_alpha with per-head Eq. 7 windows."""
    _refresh(lib.dasc_ckpt_refresh_suffix_alpha_windowed, "ckpt_refresh_suffix_alpha_windowed",
             plan, k, v, alpha, beta, tok_off, dense, dst_idx, stream, alpha=True)


def ckpt_refresh_suffix(plan: Plan, k, v, a, beta, tok_off, dense, dst_idx, stream=None) -> None:
    """Bounded-suffix refresh: replay each request's tokens from a zero
    scratch state and write the local units into dense[dst_idx[r]].
    k, v, a: bf16 CUDA tensors [T, row]; beta: fp32 [T, row]; tok_off: int64
    [n+1]; dense: [n_dense, >= dense_bytes] uint8; dst_idx: int32 [n]."""
    _refresh(lib.dasc_ckpt_refresh_suffix, "ckpt_refresh_suffix", plan, k, v, a, beta, tok_off,
             dense, dst_idx, stream)


def ckpt_unpack_refresh(plan: Plan, pool, src_slot, k, v, a, beta, tok_off, dense, dst_idx,
                        head_windows: bool = False, stream=None) -> None:
    """Load and refresh in one pass: dense[dst_idx[r]] <- what
    ckpt_unpack_zero_fill from pool[src_slot[r]] followed by the refresh
    (per-head windows if head_windows) leaves, each replayed head written
    once."""
    import torch
    n = dst_idx.numel()
    if src_slot.numel() != n or tok_off.numel() != n + 1:
        raise ValueError("src_slot must have n entries and tok_off n+1")
    T = k.shape[0]
    info = plan.info()
    for nm, t, w in (("k", k, info["k_row"]), ("v", v, info["v_row"]),
                     ("a", a, info["gate_row"]), ("beta", beta, info["beta_row"])):
        if t.dim() != 2 or t.shape[0] != T or t.shape[1] != w:
            raise ValueError(f"{nm} must be [{T}, {w}], got {tuple(t.shape)}")
    pp, ps, pn = _rows(pool, "pool")
    dp, ds, dn = _rows(dense, "dense")
    _check(lib.dasc_ckpt_unpack_refresh(
        plan._h, pp, ps, pn, _dev_ptr(src_slot, "src_slot", torch.int32),
        _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
        _dev_ptr(a, "a", torch.bfloat16), _dev_ptr(beta, "beta", torch.float32),
        _dev_ptr(tok_off, "tok_off", torch.int64), T, dp, ds, dn,
        _dev_ptr(dst_idx, "dst_idx", torch.int32), n, 1 if head_windows else 0,
        _stream_handle(stream)), "ckpt_unpack_refresh")


def ckpt_refresh_suffix_recurrent(plan: Plan, k, v, a, beta, tok_off, dense, dst_idx,
                                  stream=None) -> None:
    """As ckpt_refresh_suffix, computed token by token on the vector units
    (the recurrence's own form): the reference point for the chunked
    matrix-core kernel, several times slower."""
    _refresh(lib.dasc_ckpt_refresh_suffix_recurrent, "ckpt_refresh_suffix_recurrent", plan, k,
             v, a, beta, tok_off, dense, dst_idx, stream)


def ckpt_refresh_suffix_windowed(plan: Plan, k, v, a, beta, tok_off, dense, dst_idx,
                                 stream=None) -> None:
    """As ckpt_refresh_suffix, but each replayed head uses only the last
    min(W_lh, n_r) tokens of its request, W_lh being the head's own Eq. 7
    window (the largest W_u over its local units)."""
    _refresh(lib.dasc_ckpt_refresh_suffix_windowed, "ckpt_refresh_suffix_windowed", plan, k, v,
             a, beta, tok_off, dense, dst_idx, stream)
