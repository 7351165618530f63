"""Pins of the INT8 oracle (Eq. 10, [dasc] Appendix E.1): the page's 8.11x
and 3.88x from byte counts, closed forms of the scale and of rounding half
to even, the per-column range and error bound, and the pack / unpack round
trip against the fp32 state."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.plan import GDN, KDA
from test_oracle_plan import _kimi_rank, _layer

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_pages_8p11_capacity_and_3p88_quantization_only():
    gold = _gold("pages_numbers.json")
    # One Kimi-Linear rank keeping 3672 of its 10240 channels (184 in twelve
    # layers, 183 in eight): the fp32 ragged checkpoint then compresses
    # 2.63x (Eq. 6) and the INT8 one, 128 int8 bytes plus one fp32 scale per
    # kept channel and the bf16 conv windows, 8.11x -- both printed figures
    # from one retention.  (The retentions that give 2.63x span 8.10-8.13 in
    # INT8; a scale-less or fp32-payload mistake lands far outside.)
    per_layer = [184] * 12 + [183] * 8
    p = oracle.build_plan(_kimi_rank(per_layer), w_max=16)
    kept = sum(per_layer)
    assert kept == 3672
    assert round(p.C_ckpt, 2) == gold["kda_compression_w16"]["value"]
    lo = oracle.Int8Layout(p)
    assert lo.payload_bytes == kept * 128 and lo.scale_bytes == kept * 4
    assert lo.slot_bytes == kept * 128 + (kept * 4 + 15) // 16 * 16 + 20 * 3 * 1536 * 2
    assert round(lo.C_ckpt, 2) == gold["int8_capacity_w16"]["value"]
    # quantization only (every channel kept): fp32 temporal bytes over int8
    # payload + fp32 scales is the printed 3.88x; with the conv windows 3.53x
    q = oracle.build_plan(_kimi_rank(None), w_max=0)
    lq = oracle.Int8Layout(q)
    assert lq.payload_bytes == 20 * 4 * 128 * 128 and lq.scale_bytes == 20 * 4 * 128 * 4
    temporal_only = q.B_temp_dense / (lq.payload_bytes + lq.scale_bytes)
    assert round(temporal_only, 2) == gold["int8_quantization_only"]["value"]
    assert round(lq.C_ckpt, 2) == 3.53


def test_scale_is_column_max_over_127_and_rounding_is_half_even():
    # column max exactly 127 gives scale exactly 1.0, so the quotients are
    # the entries themselves: exact halves round to the even neighbour
    col = np.array([127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, 126.5, -127.0, 0.0], F32)
    q, s = oracle.quantize_columns(col[:, None])
    assert s[0] == F32(1.0)
    assert q[:, 0].tolist() == [127, 2, 4, -2, 0, 0, 2, 126, -127, 0]


def test_zero_and_tiny_columns_use_the_floor():
    X = np.zeros((8, 2), F32)
    X[3, 1] = F32(1e-9)                   # below the 1e-8 floor
    q, s = oracle.quantize_columns(X)
    floor = F32(F32(1e-8) / F32(127.0))
    assert s[0] == floor and s[1] == floor
    assert q[:, 0].tolist() == [0] * 8
    assert q[3, 1] == round(1e-9 / (1e-8 / 127)) == 13
    # a column whose max is exactly the floor gives the same scale and 127
    Y = np.array([[1e-8], [-5e-9]], F32)
    qy, sy = oracle.quantize_columns(Y)
    assert sy[0] == floor and qy[0, 0] == 127 and qy[1, 0] == -63


def test_scales_are_per_key_column_over_values():
    # a head [d_v, d_k] whose column k peaks at k + 1: one scale per column
    dv, dk = 6, 5
    X = np.zeros((dv, dk), F32)
    for k in range(dk):
        X[k % dv, k] = -(k + 1.0)
        X[(k + 2) % dv, k] = (k + 1.0) / 2
    q, s = oracle.quantize_columns(X)
    for k in range(dk):
        assert s[k] == F32(F32(k + 1.0) / F32(127.0))
        assert q[k % dv, k] == -127
        assert q[(k + 2) % dv, k] in (63, 64)


def test_range_and_error_bound_on_random_columns():
    rng = np.random.default_rng(5)
    X = (rng.standard_normal((128, 300)) * rng.uniform(1e-3, 1e3, 300)).astype(F32)
    q, s = oracle.quantize_columns(X)
    assert np.all(np.abs(q.astype(np.int32)).max(axis=0) == 127)
    Xh = oracle.dequantize_columns(q, s)
    err = np.abs(Xh.astype(np.float64) - X.astype(np.float64))
    bound = s.astype(np.float64)[None, :] * (0.5 + 1e-5)
    assert np.all(err <= bound)
    # dequantization is q s in fp32, exactly
    assert np.array_equal(Xh, (q.astype(F32) * s[None, :]).astype(F32))


def test_non_finite_entries_quantize_to_zero():
    X = np.array([[1.0, np.inf], [np.nan, 2.0], [-4.0, 1.0]], F32)
    q, s = oracle.quantize_columns(X)
    assert s[0] == F32(F32(4.0) / F32(127.0))      # NaN ignored by the max
    assert q[1, 0] == 0 and q[2, 0] == -127
    assert math.isinf(s[1]) and q[:, 1].tolist() == [0, 0, 0]


def test_column_maximum_skips_signaling_nans_in_any_position():
    # Eq. 10's column maximum over entries, NaN skipped: every position of a
    # quiet or signaling NaN next to a large finite maximum, in columns of the
    # head length, against the maximum written out in Python
    rng = np.random.default_rng(31)
    snan = np.array([0x7F9D2828], np.uint32).view(F32)[0]
    for nan in (snan, F32(np.nan)):
        for pos in range(0, 128, 3):
            col = (rng.standard_normal(128) * 10.0 ** rng.integers(-30, 30, 128)).astype(F32)
            col[(pos + 1) % 128] = F32(3.3e38)
            col[pos] = nan
            X = np.stack([col, col[::-1]], axis=1)
            q, s = oracle.quantize_columns(X)
            want = max(abs(float(v)) for v in col if v == v)
            assert s[0] == F32(F32(want) / F32(127.0)) and s[1] == s[0], (pos, s, want)
            assert q[pos, 0] == 0 and q[(pos + 1) % 128, 0] == 127


def _mixed_plan():
    rng = np.random.default_rng(9)
    lays = [_layer(GDN, 5, 8, 12, rng.uniform(-1, 2, 5), rng.normal(0, 1, 5), 32),
            _layer(KDA, 3, 16, 8, rng.normal(0, 1.5, 48), rng.normal(0, 1, 48), 48),
            _layer(KDA, 2, 4, 4, rng.normal(0, 1.5, 8), rng.normal(0, 1, 8), 0)]
    return oracle.build_plan(lays, w_max=4)


def test_pack_unpack_int8_round_trip():
    p = _mixed_plan()
    lo = oracle.Int8Layout(p)
    assert all(L.r > 0 for L in p.layers) and any(L.r < L.n for L in p.layers)
    assert lo.scale_base % 16 == 0 and lo.conv_base % 16 == 0
    rng = np.random.default_rng(3)
    n = 3
    dense = np.zeros((n, p.dense_bytes), np.uint8)
    dense[:, :p.B_temp_dense] = rng.standard_normal((n, p.B_temp_dense // 4)).astype(F32).view(np.uint8)
    dense[:, p.B_temp_dense:] = rng.integers(0, 256, (n, p.B_conv), dtype=np.uint8)
    pool = np.full((n, lo.slot_bytes), 0xAB, np.uint8)
    oracle.pack_int8(p, dense, [2, 0, 1], pool, [0, 1, 2])
    out = np.full_like(dense, 0xFF)
    oracle.unpack_int8_zero_fill(p, pool, [0, 1, 2], out, [2, 0, 1])
    for i in range(n):
        assert np.array_equal(out[i, p.B_temp_dense:], dense[i, p.B_temp_dense:])  # conv raw
        for li, L in enumerate(p.layers):
            a = p.temporal_off[li]
            S = dense[i, a:a + L.state_bytes].view(F32).reshape(L.n_heads, L.d_v, L.d_k)
            H = out[i, a:a + L.state_bytes].view(F32).reshape(L.n_heads, L.d_v, L.d_k)
            keep = (np.broadcast_to(L.retained[:, None, None], S.shape) if L.kind == GDN else
                    np.broadcast_to(L.retained.reshape(L.n_heads, 1, L.d_k), S.shape))
            assert np.all(H.view(np.uint32)[~keep] == 0)              # +0.0 in local units
            amax = np.abs(S).max(axis=1, keepdims=True)               # per (h, k) over v
            bound = np.broadcast_to(np.maximum(amax, 1e-8) / 127 * (0.5 + 1e-5), S.shape)
            assert np.all(np.abs(H - S)[keep] <= bound[keep])
    # the stored scales are the oracle's own per-unit scales, in unit order
    L1 = p.layers[1]
    j = 0
    u = int(L1.retained_idx[j])
    h, k = divmod(u, L1.d_k)
    S1 = dense[2, p.temporal_off[1]:p.temporal_off[1] + L1.state_bytes].view(F32).reshape(3, 8, 16)
    s_stored = pool[0, lo.scale_base + lo.s_off[1]:lo.scale_base + lo.s_off[1] + 4].view(F32)[0]
    assert s_stored == F32(F32(np.abs(S1[h][:, k]).max()) / F32(127.0))
