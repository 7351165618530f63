"""Pins for the oracle's pack and zero-fill unpack: round trip against the
mask, bijection onto the payload, raw-bit preservation, every destination
byte written (no GPU, no HIP library)."""
import numpy as np

import oracle
from workloads import GDN, KDA, Layer, special_values_f32


def _layers():
    rng = np.random.default_rng(11)
    return [
        Layer(GDN, 6, 8, 8, rng.uniform(-1, 2, 6).astype(np.float32),
              rng.normal(0, 1, 6).astype(np.float32), 32),
        Layer(KDA, 3, 8, 4, rng.normal(0, 1.5, 24).astype(np.float32),
              rng.normal(0, 1, 24).astype(np.float32), 48),
        Layer(KDA, 2, 16, 16, rng.normal(0, 1.5, 32).astype(np.float32),
              rng.normal(0, 1, 32).astype(np.float32), 0),
        Layer(GDN, 4, 4, 8, rng.uniform(-1, 2, 4).astype(np.float32),
              rng.normal(0, 1, 4).astype(np.float32), 16),
    ]


def _random_dense(plan, n, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, size=(n, plan.dense_bytes), dtype=np.uint8)


def _mask_words(plan):
    """Independent of pack: a uint32 mask over one dense checkpoint that is
    all-ones on retained units, zero on local units, all-ones on conv."""
    m = np.zeros(plan.dense_bytes // 4, dtype=np.uint32)
    for li, L in enumerate(plan.layers):
        base = plan.temporal_off[li] // 4
        for h in range(L.n_heads):
            for v in range(L.d_v):
                for k in range(L.d_k):
                    u = h if L.kind == GDN else h * L.d_k + k
                    if L.retained[u]:
                        m[base + (h * L.d_v + v) * L.d_k + k] = 0xFFFFFFFF
    m[plan.B_temp_dense // 4:] = 0xFFFFFFFF
    return m


def test_round_trip_equals_masked_state():
    for w in (0, 2, 8, 64, 1 << 30):
        plan = oracle.build_plan(_layers(), w_max=w)
        dense = _random_dense(plan, 3, w + 1)
        pool = np.zeros((4, plan.slot_bytes), dtype=np.uint8)
        oracle.pack(plan, dense, [0, 1, 2], pool, [3, 0, 2])
        out = np.full((3, plan.dense_bytes), 0xAB, dtype=np.uint8)
        oracle.unpack_zero_fill(plan, pool, [0, 2, 3], out, [1, 2, 0])
        mask = _mask_words(plan)
        for got, src in ((out[1], dense[1]), (out[2], dense[2]), (out[0], dense[0])):
            assert np.array_equal(got.view(np.uint32), src.view(np.uint32) & mask)


def test_pack_is_bijection_onto_payload():
    # Fill every unit's words with the unit's global index (+1, so zero is
    # never a label); the pool must then list the retained units in order.
    plan = oracle.build_plan(_layers(), w_max=8)
    dense = np.zeros((1, plan.dense_bytes), dtype=np.uint8)
    words = dense[0].view(np.uint32)
    label = 1
    labels = []
    for li, L in enumerate(plan.layers):
        base = plan.temporal_off[li] // 4
        S = words[base:base + L.n_heads * L.d_v * L.d_k].reshape(L.n_heads, L.d_v, L.d_k)
        for u in range(L.n):
            if L.kind == GDN:
                S[u] = label
            else:
                S[u // L.d_k, :, u % L.d_k] = label
            if L.retained[u]:
                labels.append((label, L.unit_bytes // 4))
            label += 1
    pool = np.zeros((1, plan.slot_bytes), dtype=np.uint8)
    oracle.pack(plan, dense, [0], pool, [0])
    payload = pool[0, :plan.B_temp_rag].view(np.uint32)
    expect = np.concatenate([np.full(n, lab, np.uint32) for lab, n in labels]) \
        if labels else np.zeros(0, np.uint32)
    assert np.array_equal(payload, expect)


def test_raw_bits_survive():
    plan = oracle.build_plan(_layers(), w_max=0)          # retain everything
    sv = special_values_f32()
    dense = np.zeros((1, plan.dense_bytes), dtype=np.uint8)
    w = dense[0, :plan.B_temp_dense].view(np.uint32)
    w[:] = np.resize(sv, w.shape)
    dense[0, plan.B_temp_dense:] = np.arange(plan.B_conv, dtype=np.uint8)
    pool = np.zeros((1, plan.slot_bytes), dtype=np.uint8)
    oracle.pack(plan, dense, [0], pool, [0])
    out = np.zeros_like(dense)
    oracle.unpack_zero_fill(plan, pool, [0], out, [0])
    assert np.array_equal(out, dense)


def test_unpack_overwrites_every_byte_and_zero_is_positive():
    plan = oracle.build_plan(_layers(), w_max=8)
    pool = np.zeros((1, plan.slot_bytes), dtype=np.uint8)
    out = np.full((1, plan.dense_bytes), 0xFF, dtype=np.uint8)
    oracle.unpack_zero_fill(plan, pool, [0], out, [0])
    assert not out.any()                       # all +0.0 bits, conv zero too


def test_conv_bytes_follow_payload():
    plan = oracle.build_plan(_layers(), w_max=8)
    dense = _random_dense(plan, 1, 5)
    pool = np.zeros((1, plan.slot_bytes), dtype=np.uint8)
    oracle.pack(plan, dense, [0], pool, [0])
    assert np.array_equal(pool[0, plan.B_temp_rag:], dense[0, plan.B_temp_dense:])
    assert plan.slot_bytes == plan.B_temp_rag + plan.B_conv
