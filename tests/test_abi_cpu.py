"""The C ABI without a GPU: every declared symbol is exported, the host
planner matches the oracle bit-exactly, and host-side validation rejects bad
arguments before anything reaches a device."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import recurrent_state_cache_amd as R
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dasc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dasc_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 26
    out = subprocess.run(["nm", "-D", "--defined-only", R.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b[TW]\s+(dasc_[a-z0-9_]+)\b", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(R.lib, n)


def _compare(cfg_layers, a_s, eps, w_max):
    P = R.Plan(cfg_layers, a_s, eps, w_max)
    O = oracle.build_plan(cfg_layers, a_s, eps, w_max)
    lo = oracle.Int8Layout(O)
    info = P.info()
    for l, L in enumerate(O.layers):
        r, H, w = P.units(l)
        li = P.layer(l)
        assert np.array_equal(r.astype(bool), L.retained), l
        np.testing.assert_allclose(H, L.H_s, rtol=1e-14, atol=0)
        expect_w = np.zeros(L.n, np.int64)
        expect_w[L.local_idx] = L.W_u
        assert np.array_equal(w, expect_w), l
        assert li["n_retained"] == L.r and li["n_units"] == L.n
        assert li["unit_offset"] == O.unit_off[l]
        assert li["dense_offset"] == O.temporal_off[l]
        assert li["pool_offset"] == O.pool_off[l]
        assert li["conv_dense_offset"] == O.conv_off[l]
        assert li["conv_pool_offset"] == O.pool_conv_off[l]
        assert li["unit_bytes"] == L.unit_bytes
        assert li["w_layer"] == O.W_layer[l]
        assert li["n_refresh_heads"] == len(O.refreshed_heads(l))
        assert li["int8_pool_offset"] == lo.q_off[l]
        assert li["int8_scale_offset"] == lo.scale_base + lo.s_off[l]
    assert info["n_retained"] == sum(L.r for L in O.layers)
    assert info["int8_payload_bytes"] == lo.payload_bytes
    assert info["int8_scale_bytes"] == lo.scale_bytes
    assert info["int8_slot_bytes"] == lo.slot_bytes
    assert info["c_ckpt_int8"] == lo.C_ckpt or (math.isinf(lo.C_ckpt) and math.isinf(info["c_ckpt_int8"]))
    assert info["temporal_dense_bytes"] == O.B_temp_dense
    assert info["temporal_rag_bytes"] == O.B_temp_rag
    assert info["conv_bytes"] == O.B_conv
    assert info["dense_bytes"] == O.dense_bytes and info["slot_bytes"] == O.slot_bytes
    assert info["w_replay"] == O.W_replay and info["r_max"] == O.R_max
    for key, val in (("c_temp", O.C_temp), ("c_ckpt", O.C_ckpt), ("c_temp_pad", O.C_temp_pad)):
        assert info[key] == val or (math.isinf(val) and math.isinf(info[key])), key
    return P, O


@pytest.mark.parametrize("name", ["tiny_kda", "gdn", "kda", "mixed"])
def test_plan_matches_oracle_on_configs(name):
    cfg = W.CONFIGS[name]()
    _compare(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)


@pytest.mark.parametrize("w_max", [0, 1, 4, 9, 16, 64, 1 << 30])
def test_plan_matches_oracle_across_thresholds(w_max):
    rng = np.random.default_rng(w_max % 97)
    layers = [
        W.Layer(W.GDN, 6, 8, 8, rng.uniform(-1, 2, 6).astype(np.float32),
                rng.normal(0, 1, 6).astype(np.float32), 32),
        W.Layer(W.KDA, 3, 8, 4, rng.normal(0, 1.5, 24).astype(np.float32),
                rng.normal(0, 1, 24).astype(np.float32), 48),
        W.Layer(W.KDA, 2, 16, 16, rng.normal(0, 1.5, 32).astype(np.float32),
                rng.normal(0, 1, 32).astype(np.float32), 0),
    ]
    _compare(layers, -0.3, 1e-3, w_max)


def test_exact_tie_decided_like_oracle():
    lay = W.Layer(W.GDN, 1, 4, 4, np.zeros(1, np.float32), np.full(1, 0.25, np.float32))
    P4, _ = _compare([lay], -0.25, 0.0625, 4)
    assert P4.units(0)[0][0] == 0 and P4.units(0)[1][0] == 4.0
    P3, _ = _compare([lay], -0.25, 0.0625, 3)
    assert P3.units(0)[0][0] == 1


def test_eq8_slots_from_c1_budget():
    layers = [W.Layer(W.KDA, 4, 128, 128, np.full(512, 3.0, np.float32),
                      np.zeros(512, np.float32), 3 * 1536 * 2) for _ in range(20)]
    P = R.Plan(layers, -0.3, 1e-3, 0)
    assert P.slots(694_681_600) == 127 and P.slots(694_681_600, dense=True) == 127
    assert P.slots(1000) == -1
    assert R.lib.dasc_plan_slots(None, 10, 0) == -(1 << 63)


def _desc(kind=0, H=2, dk=8, dv=8, A=None, D=None, conv=0):
    n = H if kind == 0 else H * dk
    A = np.zeros(n, np.float32) if A is None else A
    D = np.zeros(n, np.float32) if D is None else D
    return W.Layer(kind, H, dk, dv, A, D, conv)


@pytest.mark.parametrize("layer,kw", [
    (dict(kind=2), {}),
    (dict(H=0), {}),
    (dict(kind=1, dk=6), {}),
    (dict(kind=1, dk=256), {}),
    (dict(kind=1, dv=6), {}),
    (dict(conv=8), {}),
    (dict(conv=-16), {}),
    (dict(A=np.array([np.nan, 0], np.float32)), {}),
    # refresh row offsets are 32-bit: a v row of 4 x 2^30 elements is too wide
    (dict(H=4, dk=4, dv=1 << 30, A=np.zeros(4, np.float32), D=np.zeros(4, np.float32)), {}),
    (dict(D=np.array([0, np.inf], np.float32)), {}),
    ({}, dict(eps=0.0)),
    ({}, dict(eps=1.0)),
    ({}, dict(w_max=-1)),
    ({}, dict(a_s=float("nan"))),
])
def test_plan_build_rejects(layer, kw):
    args = dict(a_s=-0.3, eps=1e-3, w_max=16)
    args.update(kw)
    with pytest.raises(R.DascError) as e:
        R.Plan([_desc(**layer)], **args)
    assert e.value.code == -1
    assert R.lib.dasc_last_error().decode()


def test_null_and_empty_plan_arguments():
    h = ctypes.c_void_p()
    assert R.lib.dasc_plan_build(None, 1, -0.3, 1e-3, 16, ctypes.byref(h)) == -1
    assert R.lib.dasc_plan_build(None, 0, -0.3, 1e-3, 16, None) == -1
    assert R.lib.dasc_plan_query(None, None) == -1
    assert R.lib.dasc_plan_layer(None, 0, None) == -1
    P = R.Plan([_desc()], w_max=16)
    assert R.lib.dasc_plan_units(P._h, 5, None, None, None) == -1
    assert R.lib.dasc_plan_upload(P._h, None, 0, None) == -1
    assert R.lib.dasc_plan_destroy(None) == 0


def test_data_calls_need_uploaded_tables():
    # Nothing is launched: the host rejects the call first.
    P = R.Plan([_desc()], w_max=16)
    fake = ctypes.c_void_p(16)
    assert R.lib.dasc_ckpt_pack(P._h, fake, 4096, 1, fake, fake, 4096, 1, fake, 1, None) == -2
    assert R.lib.dasc_ckpt_unpack_zero_fill(P._h, fake, 4096, 1, fake, fake, 4096, 1, fake, 1,
                                            None) == -2
    assert R.lib.dasc_ckpt_refresh_suffix(P._h, fake, fake, fake, fake, fake, 1, fake, 4096, 1,
                                          fake, 1, None) == -2
    assert R.lib.dasc_ckpt_pack(None, fake, 4096, 1, fake, fake, 4096, 1, fake, 1, None) == -1
    s = ctypes.c_uint32()
    assert R.lib.dasc_plan_status(P._h, ctypes.byref(s), 0, None) == -2


def test_refresh_rows_reported():
    cfg = W.mixed()
    info = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max).info()
    assert info["k_row"] == 27 * 32 * 128 and info["v_row"] == 27 * 32 * 128
    assert info["gate_row"] == 14 * 32 + 13 * 32 * 128 and info["beta_row"] == 27 * 32


def _tp_compare(cfg_layers, a_s, eps, w_max, tp):
    orac = oracle.rank_plans(cfg_layers, tp, a_s, eps, w_max)
    b = oracle.plans_balance(orac)
    for rank in range(tp):
        P = R.Plan(cfg_layers, a_s, eps, w_max, tp=tp, rank=rank)
        O = orac[rank]
        ti = P.tp_info()
        M, n, t = P.tp_splits()
        assert n.tolist() == b.n and t.tolist() == b.t
        assert np.array_equal(M, b.send_units())
        ub = O.layers[0].unit_bytes
        assert (ti["tp"], ti["rank"], ti["one_store"]) == (tp, rank, 1)
        assert ti["unit_bytes"] == ub and ti["n_total"] == b.N
        assert ti["slot_units"] == b.slot_units and ti["m_remote"] == b.M_remote
        assert ti["max_local"] == max(b.n) and ti["n_local"] == b.n[rank]
        assert ti["target"] == b.t[rank] and ti["keep"] == b.keep[rank]
        assert ti["send_units"] == b.n[rank] - b.keep[rank]
        assert ti["recv_units"] == b.t[rank] - b.keep[rank]
        assert ti["slot_bytes"] == oracle.slot_bytes_tp(O, b)
        assert ti["send_bytes"] == oracle.send_bytes_tp(O, b, rank)
        # the rank's own plan is the plan of its heads
        info = P.info()
        assert info["dense_bytes"] == O.dense_bytes and info["slot_bytes"] == O.slot_bytes
        for l, L in enumerate(O.layers):
            assert np.array_equal(P.units(l)[0].astype(bool), L.retained)
    return b


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_tp_balance_matches_oracle_kda(tp):
    cfg = W.kda()
    b = _tp_compare(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max, tp)
    assert b.slot_units == math.ceil(b.N / tp)


@pytest.mark.parametrize("tp", [2, 8])
def test_tp_balance_matches_oracle_gdn(tp):
    cfg = W.gdn()
    b = _tp_compare(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max, tp)
    if tp == 8:
        assert b.M_remote > 0          # head-wise selection leaves ranks uneven


def test_plain_plan_is_rank_zero_of_one():
    cfg = W.tiny_kda()
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    ti = P.tp_info()
    assert (ti["tp"], ti["rank"], ti["keep"], ti["send_units"]) == (1, 0, ti["n_local"], 0)
    assert ti["slot_bytes"] == P.info()["slot_bytes"]


def test_tp_build_rejects():
    cfg = W.tiny_kda()                  # 4 heads
    with pytest.raises(R.DascError):
        R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max, tp=3, rank=0)
    with pytest.raises(R.DascError):
        R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max, tp=2, rank=2)
    mixed = W.mixed(n_ckpt=4, n_req=4)  # GDN and KDA units differ in size
    with pytest.raises(R.DascError) as e:
        R.Plan(mixed.layers, mixed.a_s, mixed.eps, mixed.w_max, tp=2, rank=0)
    assert e.value.code == -5


def test_every_data_call_needs_uploaded_tables():
    # The newer entry points reject a plan whose tables are not on a device
    # (DASC_ENOTUPLOADED) or a null plan (DASC_EINVAL) before any launch.
    P = R.Plan([_desc()], w_max=16)
    f = ctypes.c_void_p(16)
    L = R.lib
    calls = {
        "pack_int8": lambda h: L.dasc_ckpt_pack_int8(h, f, 4096, 1, f, f, 4096, 1, f, 1, None),
        "unpack_int8": lambda h: L.dasc_ckpt_unpack_int8_zero_fill(h, f, 4096, 1, f, f, 4096, 1,
                                                                 f, 1, None),
        "refresh_windowed": lambda h: L.dasc_ckpt_refresh_suffix_windowed(h, f, f, f, f, f, 1, f,
                                                                          4096, 1, f, 1, None),
        "refresh_recurrent": lambda h: L.dasc_ckpt_refresh_suffix_recurrent(h, f, f, f, f, f, 1,
                                                                            f, 4096, 1, f, 1,
                                                                            None),
        "refresh_alpha": lambda h: L.dasc_ckpt_refresh_suffix_alpha(h, f, f, f, f, f, 1, f,
                                                                    4096, 1, f, 1, None),
        "refresh_alpha_windowed": lambda h: L.dasc_ckpt_refresh_suffix_alpha_windowed(
            h, f, f, f, f, f, 1, f, 4096, 1, f, 1, None),
        "pack_tp": lambda h: L.dasc_ckpt_pack_tp(h, f, 4096, 1, f, f, 4096, 1, f, f, 4096, 1, f,
                                                 1, None),
        "unpack_tp": lambda h: L.dasc_ckpt_unpack_tp_zero_fill(h, f, 4096, 1, f, f, 4096, 1, f,
                                                               f, 4096, 1, f, 1, None),
        "unpack_refresh": lambda h: L.dasc_ckpt_unpack_refresh(h, f, 4096, 1, f, f, f, f, f, f, 1,
                                                               f, 4096, 1, f, 1, 0, None),
    }
    for name, call in calls.items():
        assert call(P._h) == -2, name
        assert call(None) == -1, name


def test_tp_calls_reject_a_mixed_store_plan():
    # GDN and KDA layers have units of different sizes: no balancing
    cfg = W.mixed(n_ckpt=2, n_req=2)
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    assert P.tp_info()["one_store"] == 0
    f = ctypes.c_void_p(16)
    assert R.lib.dasc_ckpt_pack_tp(P._h, f, 4096, 1, f, f, 4096, 1, f, f, 4096, 1, f, 1,
                                   None) == -5


def test_plan_launches():
    # dasc_plan_launches: launches of at most 16 pairs (INT8 pack: 32),
    # raised where a launch would hold too few workgroups, evened out
    cfg = W.kda(n_ckpt=64, n_req=2, window=8)
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    for mover in ("pack", "unpack", "pack_int8", "unpack_int8"):
        for n in (1, 5, 16, 17, 64, 100, 512):
            nl, per = P.launches(mover, n)
            assert nl >= 1 and per >= 1 and (nl - 1) * per < n <= nl * per, (mover, n, nl, per)
            base = 32 if mover == "pack_int8" else 16
            assert nl <= -(-n // base)  # the workgroup minimum only merges launches
        assert P.launches(mover, 0) == (0, 0)
    assert P.launches("pack", 64) == (4, 16)
    # the INT8 unpack list holds few pieces here: launches of 22 + 21 + 21
    assert P.launches("unpack_int8", 64) == (3, 22)
    assert P.launches("pack_tp", 64)[0] >= 1  # TP = 1: the plain slot
    with pytest.raises(R.DascError):
        P.launches("unpack", -1)
    h = ctypes.c_int32(0)
    assert R.lib.dasc_plan_launches(P._h, 9, 4, ctypes.byref(h), ctypes.byref(h)) != 0
    Pt = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max, tp=8, rank=3)
    nl, per = Pt.launches("unpack_tp", 64)
    assert nl * per >= 64
