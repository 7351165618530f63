"""Pins for the oracle's bounded-suffix refresh: brute force against the
printed matrix form, the delta rule's exact-recall and pure-decay closed
forms, the contraction bound, and the gate and row-layout wiring of
refresh_expected (no GPU, no HIP library)."""
import math

import numpy as np
import pytest

import oracle
from workloads import GDN, KDA, Layer


def _rand_inputs(rng, W, dk, dv, alpha_lo=0.2):
    al = rng.uniform(alpha_lo, 1.0, (W, dk))
    be = rng.uniform(0.0, 1.0, W)
    ks = rng.normal(0, 1, (W, dk))
    ks /= np.linalg.norm(ks, axis=1, keepdims=True)
    vs = rng.normal(0, 1, (W, dv))
    return al, be, ks, vs


def test_rank1_matches_printed_matrix_form():
    rng = np.random.default_rng(20)
    for dk, dv in ((4, 4), (8, 5), (16, 16)):
        al, be, ks, vs = _rand_inputs(rng, 12, dk, dv)
        S0 = rng.normal(0, 1, (dv, dk))
        a = oracle.replay_rank1(al, be, ks, vs, S0)
        b = oracle.replay_dense(al, be, ks, vs, S0)
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.linalg.norm(b))
        # unnormalised keys and beta up to 2 too
        ks2 = rng.normal(0, 1, (12, dk))
        be2 = rng.uniform(0, 2, 12)
        a = oracle.replay_rank1(al, be2, ks2, vs, S0)
        b = oracle.replay_dense(al, be2, ks2, vs, S0)
        assert np.max(np.abs(a - b)) <= 1e-10 * max(1.0, np.linalg.norm(b))


def test_gdn_scalar_decay_equals_broadcast():
    rng = np.random.default_rng(21)
    W, d = 10, 8
    a_scalar = rng.uniform(0.3, 1.0, W)
    _, be, ks, vs = _rand_inputs(rng, W, d, d)
    S = oracle.replay_rank1(np.repeat(a_scalar[:, None], d, 1), be, ks, vs)
    T = np.zeros((d, d))
    for t in range(W):        # S <- a S (I - b k k^T) + b v k^T, scalar a
        k, v = ks[t][:, None], vs[t][:, None]
        T = a_scalar[t] * T @ (np.eye(d) - be[t] * k @ k.T) + be[t] * v @ k.T
    np.testing.assert_allclose(S, T, atol=1e-12)


def _exact_unit_keys(rng, d, W):
    """Keys with exactly unit norm in bf16 and float64: one-hot, +-1/2 on 4
    coordinates, or +-1/4 on 16 coordinates."""
    ks = np.zeros((W, d))
    for t in range(W):
        m = [1, 4, 16][t % 3] if d >= 16 else [1, 4][t % 2]
        idx = rng.choice(d, m, replace=False)
        ks[t, idx] = rng.choice([-1.0, 1.0], m) / math.sqrt(m)
    return ks


def test_beta_one_recalls_last_value_exactly():
    # With beta = 1 and |k| = 1: S_t k_t = v_t, whatever alpha and S_{t-1}.
    rng = np.random.default_rng(22)
    d = 16
    ks = _exact_unit_keys(rng, d, 40)
    al = rng.uniform(0.01, 1.0, (40, d))
    vs = rng.normal(0, 1, (40, d))
    S = rng.normal(0, 1, (d, d))
    for t in range(40):
        S = oracle.delta_rule_step(S, al[t], np.float64(1.0), ks[t], vs[t])
        np.testing.assert_allclose(S @ ks[t], vs[t], atol=1e-12)


def test_beta_zero_is_pure_column_decay():
    # beta = 0 and constant alpha: S_W = S_0 Diag(alpha)^W, column by column.
    rng = np.random.default_rng(23)
    d, W = 8, 256
    alpha = rng.uniform(0.9, 0.999, d)
    S0 = rng.normal(0, 1, (d, d))
    ks = rng.normal(0, 1, (W, d))
    vs = rng.normal(0, 1, (W, d))
    S = oracle.replay_rank1(np.tile(alpha, (W, 1)), np.zeros(W), ks, vs, S0)
    expect = np.array([[S0[i, j] * alpha[j] ** W for j in range(d)] for i in range(d)])
    np.testing.assert_allclose(S, expect, rtol=1e-12)


def test_one_hot_write_then_decay_closed_form():
    # From zero: token j (j < d) writes v_j into column j with k = e_j and
    # beta = 1; every later token multiplies column j by its alpha[j]; then
    # W - d tokens with beta = 0 and constant alpha.
    rng = np.random.default_rng(24)
    d, W = 8, 40
    al = rng.uniform(0.5, 1.0, (W, d))
    al[d:] = al[d]
    be = np.concatenate([np.ones(d), np.zeros(W - d)])
    ks = np.concatenate([np.eye(d), rng.normal(0, 1, (W - d, d))])
    vs = rng.normal(0, 1, (W, d))
    S = oracle.replay_rank1(al, be, ks, vs)
    expect = np.zeros((d, d))
    for j in range(d):
        f = 1.0
        for t in range(j + 1, W):
            f *= al[t, j]
        expect[:, j] = vs[j] * f
    np.testing.assert_allclose(S, expect, rtol=1e-13, atol=1e-15)


def test_orthonormal_keys_store_every_pair():
    # alpha = 1, beta = 1, orthonormal keys: S = sum_j v_j k_j^T, so S k_j = v_j.
    rng = np.random.default_rng(25)
    d = 12
    Q, _ = np.linalg.qr(rng.normal(0, 1, (d, d)))
    ks = Q.T
    vs = rng.normal(0, 1, (d, d))
    S = oracle.replay_rank1(np.ones((d, d)), np.ones(d), ks, vs)
    for j in range(d):
        np.testing.assert_allclose(S @ ks[j], vs[j], atol=1e-12)


def test_contraction_bound():
    # |S_t|_F <= max(alpha_t) |S_{t-1}|_F + beta_t |v_t| for |k_t| = 1,
    # beta in [0, 1] (the transition's 2-norm is at most max alpha).
    rng = np.random.default_rng(26)
    d = 16
    al, be, ks, vs = _rand_inputs(rng, 200, d, d, alpha_lo=0.0)
    S = rng.normal(0, 3, (d, d))
    for t in range(200):
        Sn = oracle.delta_rule_step(S, al[t], be[t], ks[t], vs[t])
        bound = al[t].max() * np.linalg.norm(S) + be[t] * np.linalg.norm(vs[t])
        assert np.linalg.norm(Sn) <= bound * (1 + 1e-12)
        S = Sn


def _bf16_bits(x):
    """float -> bf16 bits (round to nearest even), for exactly representable
    test values only."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((f & 0xFFFF) == 0)
    return (f >> 16).astype(np.uint16)


@pytest.mark.parametrize("dk,dv", [(8, 8), (8, 4), (4, 12)])
def test_refresh_expected_wiring_gate_and_rows(dk, dv):
    # Two layers (GDN then KDA) share one token row.  Token logits a_t = -1/4
    # and dt_bias = 1/4 make softplus(a_t + dt_bias) = ln 2 exactly, so each
    # unit decays by exp(-exp(A_log) ln 2) per token: 1/2 where A_log = 0.
    gdn = Layer(GDN, 2, dk, dv, np.array([0.0, 1.0], np.float32), np.full(2, 0.25, np.float32))
    A = np.zeros(2 * dk, np.float32)
    A[:3] = -9.0                               # head 0: channels 0..2 retained
    kda = Layer(KDA, 2, dk, dv, A, np.full(2 * dk, 0.25, np.float32))
    plan = oracle.build_plan([gdn, kda], a_s=-0.3, w_max=64)
    assert list(plan.refreshed_heads(0)) == [0, 1]
    assert list(plan.refreshed_heads(1)) == [0, 1]
    assert list(plan.layers[1].retained_idx) == [0, 1, 2]
    W = 2 * dk + 1
    rng = np.random.default_rng(27)
    kw, vw, gw, bw = 4 * dk, 4 * dv, 2 + 2 * dk, 4
    k = np.zeros((W, kw), np.float32)
    v = rng.integers(-8, 8, (W, vw)).astype(np.float32)     # bf16-exact
    a = np.full((W, gw), -0.25, np.float32)
    beta = np.zeros((W, bw), np.float32)
    # rows: layer 0 (GDN) head h at h*d, layer 1 (KDA) head h at 2d + h*d
    for t in range(dk):
        for h in range(4):
            k[t, h * dk + t] = 1.0
        beta[t, :] = 1.0
    out = oracle.refresh_expected(plan, _bf16_bits(k), _bf16_bits(v), _bf16_bits(a),
                                  beta, np.array([0, W]))
    for li in (0, 1):
        for h in (0, 1):
            S = out[(0, li, h)]
            assert S.shape == (dv, dk)
            c0 = (2 * li + h) * dv
            vv = v[:, c0:c0 + dv].astype(np.float64)
            for j in range(dk):
                A_u = gdn.A_log[h] if li == 0 else kda.A_log[h * dk + j]
                dec = math.exp(-math.exp(float(A_u)) * math.log(2.0))
                # column j written by token j, then decayed by tokens j+1..W-1
                np.testing.assert_allclose(S[:, j], vv[j] * dec ** (W - 1 - j), rtol=1e-12)


def test_refresh_expected_respects_windows():
    d = 4
    lay = Layer(KDA, 1, d, d, np.full(d, 3.0, np.float32), np.zeros(d, np.float32))
    plan = oracle.build_plan([lay], w_max=16)
    rng = np.random.default_rng(28)
    T = 7
    k = _bf16_bits(np.eye(d)[rng.integers(0, d, T)].astype(np.float32))
    v = _bf16_bits(rng.integers(-4, 4, (T, d)).astype(np.float32))
    a = _bf16_bits(np.zeros((T, d), np.float32))
    beta = np.ones((T, 1), np.float32)
    out = oracle.refresh_expected(plan, k, v, a, beta, np.array([0, 3, 3, 7]))
    assert (1, 0, 0) in out and not np.any(out[(1, 0, 0)])          # W = 0
    solo = oracle.refresh_expected(plan, k[3:], v[3:], a[3:], beta[3:], np.array([0, 4]))
    np.testing.assert_array_equal(out[(2, 0, 0)], solo[(0, 0, 0)])


def _windowed_plan():
    # a_s + dt_bias = 0: H_s = log2(1000) / exp(A_log).  KDA heads with
    # windows 8, 16 and 4 (one fully retained head), GDN heads 8, 4, 16.
    lg = math.log2(1000.0)
    kda_H = [3.0, 5.0, 100.0, 2.0, 50.0, 60.0, 70.0, 80.0, 12.0, 0.5, 7.0, 16.5,
             1.5, 2.5, 3.5, 3.9]
    gdn_H = [6.0, 20.0, 2.2, 9.0]
    A_k = np.array([math.log(lg / h) for h in kda_H], np.float32)
    A_g = np.array([math.log(lg / h) for h in gdn_H], np.float32)
    return oracle.build_plan([Layer(KDA, 4, 4, 4, A_k, np.full(16, 0.25, np.float32)),
                              Layer(GDN, 4, 4, 4, A_g, np.full(4, 0.25, np.float32))],
                             a_s=-0.25, eps=1e-3, w_max=16)


def test_head_windows_replay_each_heads_last_tokens():
    plan = _windowed_plan()
    rng = np.random.default_rng(29)
    lens = [0, 3, 4, 5, 8, 9, 16, 23]
    tok = np.concatenate([[0], np.cumsum(lens)])
    T = int(tok[-1])
    trunc = lambda x: (x.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    k = _bf16_bits(trunc(rng.normal(0, 0.5, (T, 32))))
    v = _bf16_bits(trunc(rng.normal(0, 1, (T, 32))))
    a = _bf16_bits(trunc(rng.normal(0, 1, (T, 20))))
    beta = rng.uniform(0, 1, (T, 8)).astype(np.float32)
    win = oracle.refresh_expected(plan, k, v, a, beta, tok, head_windows=True)
    full = oracle.refresh_expected(plan, k, v, a, beta, tok)
    assert win.keys() == full.keys()
    for (r, li, h), S in win.items():
        W = {(0, 0): 8, (0, 2): 16, (0, 3): 4, (1, 0): 8, (1, 2): 4, (1, 3): 16}[(li, h)]
        t1 = int(tok[r + 1])
        t0 = max(int(tok[r]), t1 - W)
        # the same head replayed alone over its last W tokens
        solo = oracle.refresh_expected(plan, k, v, a, beta, np.array([t0, t1]), layers=[li],
                                       heads=[h])
        np.testing.assert_array_equal(S, solo[(0, li, h)])
        if lens[r] <= W:
            np.testing.assert_array_equal(S, full[(r, li, h)])
        else:
            assert not np.array_equal(S, full[(r, li, h)])
        if lens[r] == 0:
            assert not np.any(S)


@pytest.mark.parametrize("dk,dv", [(8, 8), (8, 4), (4, 12)])
def test_refresh_expected_alpha_rows(dk, dv):
    # Decays given directly (Eq. 1 as written), one per head for GDN and one
    # per channel for KDA, read from their own columns of the alpha row: a
    # one-hot write phase (beta = 1, k = e_j at token j) then beta = 0, so
    # column j of every head's state is v_j times the product of the decays
    # that column sees after token j.  Every head and channel gets its own
    # decay sequence, so a wrong row offset, a GDN decay read per channel or
    # a KDA decay taken per head would change the result.
    gdn = Layer(GDN, 2, dk, dv, np.zeros(2, np.float32), np.full(2, 0.25, np.float32))
    A = np.zeros(2 * dk, np.float32)
    A[:3] = -9.0                               # KDA head 0: channels 0..2 retained
    kda = Layer(KDA, 2, dk, dv, A, np.full(2 * dk, 0.25, np.float32))
    plan = oracle.build_plan([gdn, kda], a_s=-0.3, w_max=64)
    W = 2 * dk + 3
    rng = np.random.default_rng(31)
    kw, vw, gw, bw = 4 * dk, 4 * dv, 2 + 2 * dk, 4
    k = np.zeros((W, kw), np.float32)
    v = rng.integers(-8, 8, (W, vw)).astype(np.float32)
    alpha = rng.uniform(0.5, 1.0, (W, gw)).astype(np.float32)
    beta = np.zeros((W, bw), np.float32)
    for t in range(dk):
        for h in range(4):
            k[t, h * dk + t] = 1.0
        beta[t, :] = 1.0
    out = oracle.refresh_expected(plan, _bf16_bits(k), _bf16_bits(v), None, beta,
                                  np.array([0, W]), alpha=alpha)
    for li in (0, 1):
        for h in (0, 1):
            S = out[(0, li, h)]
            c0 = (2 * li + h) * dv
            vv = v[:, c0:c0 + dv].astype(np.float64)
            for j in range(dk):
                col = h if li == 0 else 2 + h * dk + j       # the unit's alpha column
                f = np.prod(alpha[j + 1:, col].astype(np.float64))
                np.testing.assert_allclose(S[:, j], vv[j] * f, rtol=1e-12)


def test_refresh_expected_alpha_matches_gate_when_alpha_is_the_gate():
    # The two ways of giving the decays agree when the alpha row holds the
    # gate's decays exactly: a_t = -1/4, dt_bias = 1/4, A_log = 0 makes every
    # decay exactly 1/2 by Eq. 2, and an alpha row of 1/2 gives the same
    # states bit for bit.
    d = 8
    kda = Layer(KDA, 2, d, d, np.zeros(2 * d, np.float32), np.full(2 * d, 0.25, np.float32))
    gdn = Layer(GDN, 2, d, d, np.zeros(2, np.float32), np.full(2, 0.25, np.float32))
    plan = oracle.build_plan([kda, gdn], a_s=-0.3, w_max=64)
    rng = np.random.default_rng(32)
    T = 13
    trunc = lambda x: (x.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    k = _bf16_bits(trunc(rng.normal(0, 0.4, (T, 4 * d))))
    v = _bf16_bits(trunc(rng.normal(0, 1, (T, 4 * d))))
    a = _bf16_bits(np.full((T, 2 * d + 2), -0.25, np.float32))
    beta = rng.uniform(0, 1, (T, 4)).astype(np.float32)
    tok = np.array([0, 5, T])
    via_gate = oracle.refresh_expected(plan, k, v, a, beta, tok)
    direct = oracle.refresh_expected(plan, k, v, None, beta, tok,
                                     alpha=np.full((T, 2 * d + 2), 0.5, np.float32))
    assert via_gate.keys() == direct.keys()
    for key in via_gate:
        np.testing.assert_array_equal(via_gate[key], direct[key])
