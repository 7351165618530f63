"""Pins for the oracle's static plan: closed forms, printed numbers,
invariants and special cases (no GPU, no HIP library)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import GDN, KDA, Layer

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _py_softplus(x: float) -> float:
    # textbook ln(1 + e^x), scalar Python math
    return math.log1p(math.exp(x))


def _layer(kind, H, dk, dv, A, D, conv=0):
    return Layer(kind, H, dk, dv, np.asarray(A, np.float32), np.asarray(D, np.float32), conv)


def test_half_decay_gives_log2_1000():
    # A_log = 0 and a_s + dt_bias = 0 exactly: softplus(0) = ln 2, so the
    # static decay is 1/2 per token and the horizon is log2(1/eps) tokens.
    lay = _layer(GDN, 1, 4, 4, [0.0], [0.25])
    p = oracle.build_plan([lay], a_s=-0.25, eps=1e-3, w_max=9)
    assert p.layers[0].g[0] == pytest.approx(-math.log(2.0), rel=1e-15)
    assert p.layers[0].H_s[0] == pytest.approx(math.log2(1000.0), rel=1e-15)
    assert p.layers[0].retained[0]          # 9.97 > 9
    p10 = oracle.build_plan([lay], a_s=-0.25, eps=1e-3, w_max=10)
    assert not p10.layers[0].retained[0]    # 9.97 <= 10


def test_softplus_matches_textbook_and_is_stable():
    xs = np.linspace(-30, 30, 241)
    ref = np.array([_py_softplus(float(x)) for x in xs])
    np.testing.assert_allclose(oracle.softplus(xs), ref, rtol=1e-14, atol=0)
    # softplus(x) - softplus(-x) = x, and no overflow far out
    big = np.array([-800.0, -60.0, 60.0, 800.0])
    sp = oracle.softplus(big)
    assert np.all(np.isfinite(sp))
    np.testing.assert_allclose(oracle.softplus(xs) - oracle.softplus(-xs), xs, atol=1e-12)
    assert sp[3] == 800.0 and 0.0 <= sp[0] < 1e-300


def test_gate_inverts_to_chosen_decay():
    # Invert Eq. 2 by hand: A_log = ln(-ln(alpha) / softplus(a_s + dt_bias)),
    # then the oracle's exp(g) must give back alpha.
    rng = np.random.default_rng(0)
    alphas = rng.uniform(0.01, 0.999, 200)
    dts = rng.normal(0, 1, 200).astype(np.float32)
    A = np.array([math.log(-math.log(a) / _py_softplus(-0.3 + float(d)))
                  for a, d in zip(alphas, dts)], dtype=np.float32)
    g = oracle.gate_log_decay(A, dts, -0.3)
    np.testing.assert_allclose(np.exp(g), alphas, rtol=2e-6)


def test_horizon_is_where_decay_reaches_eps():
    rng = np.random.default_rng(1)
    A = rng.normal(0, 1.5, 500).astype(np.float32)
    D = rng.normal(0, 1, 500).astype(np.float32)
    g = oracle.gate_log_decay(A, D, -0.3)
    H = oracle.horizon(g, 1e-3)
    assert np.all(g < 0) and np.all(H > 0)
    # the defining property: (e^g)^H = eps
    np.testing.assert_allclose(np.exp(g) ** H, 1e-3, rtol=1e-9)


def test_static_logit_lengthens_horizons():
    # a = -0.3 gives slower decay and longer horizons than a = 0 (§3.3).
    rng = np.random.default_rng(2)
    A = rng.normal(0, 1, 300).astype(np.float32)
    D = rng.normal(0, 1, 300).astype(np.float32)
    H03 = oracle.horizon(oracle.gate_log_decay(A, D, -0.3), 1e-3)
    H0 = oracle.horizon(oracle.gate_log_decay(A, D, 0.0), 1e-3)
    assert np.all(H03 > H0)


def test_pages_median_decays_against_16_token_cutoff():
    # Retain iff the static one-step decay exceeds eps^(1/W_max): at
    # W_max = 16 that is 0.6494.  Kimi-Linear's median 0.471 falls below it,
    # Qwen3-Next's 0.969 and Kimi-K3's 0.942 above it.
    gold = _gold("pages_numbers.json")["median_static_alpha"]
    thr = 1e-3 ** (1 / 16)
    assert abs(thr - 0.64938) < 1e-5
    for name, alpha in [(k, v) for k, v in gold.items() if k != "cite"]:
        A = math.log(-math.log(alpha) / _py_softplus(0.0))
        lay = _layer(GDN, 1, 4, 4, [A], [0.3])
        p = oracle.build_plan([lay], a_s=-0.3, eps=1e-3, w_max=16)
        assert p.layers[0].retained[0] == (alpha > thr), name
        assert p.layers[0].H_s[0] == pytest.approx(math.log(1e-3) / math.log(alpha), rel=1e-6)


def test_mask_equals_decay_threshold_rule():
    rng = np.random.default_rng(3)
    H, dk = 8, 32
    A = rng.normal(0, 1.5, H * dk).astype(np.float32)
    D = rng.normal(0, 1, H * dk).astype(np.float32)
    for w in (4, 16, 64, 512):
        p = oracle.build_plan([_layer(KDA, H, dk, 16, A, D)], w_max=w)
        alpha = np.array([math.exp(-math.exp(float(a)) * _py_softplus(-0.3 + float(d)))
                          for a, d in zip(A, D)])
        thr = 1e-3 ** (1.0 / w)
        far = np.abs(alpha - thr) > 1e-9
        assert np.array_equal(p.layers[0].retained[far], (alpha > thr)[far])


def test_exact_tie_is_omitted():
    # eps = 2^-4 and decay 1/2 make H_s exactly 4.0 in float64; strict ">"
    # omits the unit at W_max = 4 and retains it at W_max = 3.
    lay = _layer(GDN, 1, 4, 4, [0.0], [0.25])
    p4 = oracle.build_plan([lay], a_s=-0.25, eps=0.0625, w_max=4)
    assert p4.layers[0].H_s[0] == 4.0
    assert not p4.layers[0].retained[0]
    assert p4.W_replay == 4
    p3 = oracle.build_plan([lay], a_s=-0.25, eps=0.0625, w_max=3)
    assert p3.layers[0].retained[0] and p3.W_replay == 0


def test_eq7_windows_worked_by_hand():
    for c in _gold("eq7_windows.json")["cases"]:
        assert oracle.replay_window(c["H_s"], c["w_max"]) == c["W_u"], c


def test_replay_window_is_max_over_local_units():
    rng = np.random.default_rng(4)
    lay = _layer(KDA, 4, 16, 16, rng.normal(0, 1.5, 64), rng.normal(0, 1, 64))
    p = oracle.build_plan([lay], w_max=64)
    L = p.layers[0]
    ws = [oracle.replay_window(float(L.H_s[u]), 64) for u in range(64) if not L.retained[u]]
    assert p.W_replay == max(ws)
    assert all(w in (4, 8, 16, 32, 64) for w in ws)


def _mixed_small():
    rng = np.random.default_rng(5)
    return [
        _layer(GDN, 6, 8, 8, rng.uniform(-1, 2, 6), rng.normal(0, 1, 6), 32),
        _layer(KDA, 3, 8, 4, rng.normal(0, 1.5, 24), rng.normal(0, 1, 24), 48),
        _layer(KDA, 2, 16, 16, rng.normal(0, 1.5, 32), rng.normal(0, 1, 32), 0),
        _layer(GDN, 4, 4, 8, rng.uniform(-1, 2, 4), rng.normal(0, 1, 4), 16),
    ]


def test_ragged_offsets_order_and_bytes():
    p = oracle.build_plan(_mixed_small(), w_max=8)
    o = 0
    pb = 0
    for li, L in enumerate(p.layers):
        assert p.unit_off[li] == o
        assert p.pool_off[li] == pb
        assert np.all(np.diff(L.retained_idx) > 0)           # ascending
        assert len(L.retained_idx) + len(L.local_idx) == L.n
        o += L.r
        pb += L.r * L.unit_bytes
    assert p.unit_off[-1] == o
    assert p.B_temp_rag == pb
    assert p.B_temp_dense == sum(L.n_heads * L.d_v * L.d_k * 4 for L in p.layers)
    assert p.B_conv == 32 + 48 + 0 + 16
    assert p.conv_off[0] == p.B_temp_dense and p.pool_conv_off[0] == p.B_temp_rag


def test_ragged_vs_padded_gain_identity():
    # Appendix B: C_rag / C_pad = R_max / r_bar; C_rag = sum n / sum r.
    p = oracle.build_plan(_mixed_small(), w_max=8)
    assert p.C_temp_rag / p.C_temp_pad == pytest.approx(p.R_max / p.r_bar, rel=1e-15)
    assert p.C_temp_rag == pytest.approx(p.C_temp, rel=1e-15)


def test_w_max_zero_is_dense_and_huge_w_max_keeps_none():
    p0 = oracle.build_plan(_mixed_small(), w_max=0)
    assert all(L.r == L.n for L in p0.layers)
    assert p0.C_ckpt == 1.0 and p0.W_replay == 0
    pinf = oracle.build_plan(_mixed_small(), w_max=1 << 40)
    assert all(L.r == 0 for L in pinf.layers)
    assert pinf.C_ckpt == pytest.approx(p0.dense_bytes / p0.B_conv)


def _kimi_rank(retained_per_layer=None):
    """One TP8 rank of Kimi-Linear: 20 KDA layers x 4 heads x 128 x 128,
    3 conv positions x 1536 channels bf16 per layer."""
    layers = []
    for l in range(20):
        n = 4 * 128
        A = np.full(n, 3.0, np.float32)                # fast decay: local
        if retained_per_layer is not None:
            A[:retained_per_layer[l]] = -8.0            # slow decay: retained
        layers.append(_layer(KDA, 4, 128, 128, A, np.zeros(n), 3 * 1536 * 2))
    return layers


def test_c1_budget_decomposition_and_eq8():
    gold = _gold("pages_numbers.json")
    kimi = gold["kimi_kda_rank_budget_bytes"]
    p = oracle.build_plan(_kimi_rank(), w_max=0)         # Dense: W_max = 0
    assert p.dense_bytes * kimi["dense_slots"] == kimi["value"]
    assert oracle.slots_eq8(kimi["value"], p.slot_bytes) == kimi["deployable_slots"]
    qwen = gold["qwen_gdn_rank_budget_bytes"]
    layers = [_layer(GDN, 4, 128, 128, np.zeros(4), np.zeros(4), 3 * 1024 * 2)
              for _ in range(36)]
    q = oracle.build_plan(layers, w_max=0)
    assert q.dense_bytes * qwen["dense_slots"] == qwen["value"]
    assert oracle.slots_eq8(qwen["value"], q.slot_bytes) == qwen["deployable_slots"]


def test_kimi_linear_state_size():
    # 20 layers x 32 heads x 128 x 128 fp32 = 41.9 MB per request.
    gold = _gold("pages_numbers.json")["kimi_linear_state_bytes_per_request"]
    layers = [_layer(KDA, 32, 128, 128, np.zeros(4096), np.zeros(4096)) for _ in range(20)]
    p = oracle.build_plan(layers, w_max=16)
    assert round(p.B_temp_dense / 1e6, 1) == gold["value_mb"]


def test_eq6_reproduces_kda_2p63_and_eq8_2p64():
    # Retaining ~35.84% of each rank's channels (183 or 184 of 512 per
    # layer) gives the pages' 2.63x checkpoint compression by Eq. 6, and
    # Eq. 8 turns it into a 2.64x slot count against 127 dense slots.
    gold = _gold("pages_numbers.json")
    per_layer = [183 if l % 2 == 0 else 184 for l in range(20)]
    p = oracle.build_plan(_kimi_rank(per_layer), w_max=16)
    assert [L.r for L in p.layers] == per_layer
    assert round(p.C_ckpt, 2) == gold["kda_compression_w16"]["value"]
    budget = gold["kimi_kda_rank_budget_bytes"]["value"]
    ratio = oracle.slots_eq8(budget, p.slot_bytes) / 127
    assert round(ratio, 2) == gold["kda_compression_w16"]["slot_ratio_p1"]
    # and the layer-median retained fraction 0.360 lands within 0.015 of it
    frac = gold["kda_compression_w16"]["layer_median_retained_fraction"]
    med = [int(round(frac * 512))] * 20
    pm = oracle.build_plan(_kimi_rank(med), w_max=16)
    assert abs(pm.C_ckpt - 2.63) < 0.015


def test_refreshed_heads_rule():
    H, dk = 4, 8
    A = np.full(H * dk, 3.0)        # local everywhere ...
    A[0:dk] = -8.0                  # ... head 0 fully retained
    A[dk:dk + 3] = -8.0             # head 1 mixed
    p = oracle.build_plan([_layer(KDA, H, dk, 8, A, np.zeros(H * dk))], w_max=16)
    assert list(p.refreshed_heads(0)) == [1, 2, 3]
    g = oracle.build_plan([_layer(GDN, 4, 8, 8, [-8.0, 3.0, -8.0, 3.0], np.zeros(4))], w_max=16)
    assert list(g.refreshed_heads(0)) == [1, 3]


def test_head_window_worked_by_hand():
    # a_s + dt_bias = 0 makes softplus = ln 2, so H_s = log2(1000) / exp(A_log)
    # and A_log = ln(log2(1000) / H) puts each horizon where the table says.
    # Per head, W_lh = max over local units of clamp(next_pow2(H_s), 4, 16),
    # worked by hand (Eq. 7 per head; 0 = no local unit, head not replayed).
    lg = math.log2(1000.0)
    kda_H = [[3.0, 5.0, 100.0, 2.0],      # W_u 4, 8, retained, 4      -> 8
             [50.0, 60.0, 70.0, 80.0],    # all retained               -> 0
             [12.0, 0.5, 7.0, 16.5],      # 16, 4, 8, retained         -> 16
             [1.5, 2.5, 3.5, 3.9]]        # 4, 4, 4, 4                 -> 4
    gdn_H = [6.0, 20.0, 2.2, 9.0]         # 8, retained, 4, 16
    A_k = [math.log(lg / h) for row in kda_H for h in row]
    A_g = [math.log(lg / h) for h in gdn_H]
    kda = _layer(KDA, 4, 4, 4, A_k, np.full(16, 0.25))
    gdn = _layer(GDN, 4, 4, 4, A_g, np.full(4, 0.25))
    p = oracle.build_plan([kda, gdn], a_s=-0.25, eps=1e-3, w_max=16)
    assert [p.head_window(0, h) for h in range(4)] == [8, 0, 16, 4]
    assert [p.head_window(1, h) for h in range(4)] == [8, 0, 4, 16]
    assert list(p.refreshed_heads(0)) == [0, 2, 3]
    assert list(p.refreshed_heads(1)) == [0, 2, 3]
    assert p.W_layer == [16, 16] and p.W_replay == 16
