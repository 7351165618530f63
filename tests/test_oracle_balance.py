"""Pins for the oracle's TP storage balancing ([dasc] §4.3, Appendix
B.1(b)): hand-worked assignments, brute-force minimality of the moved units,
the target invariants, and store / load round trips (no GPU, no HIP
library)."""
import itertools
import math

import numpy as np
import pytest

import oracle
from workloads import GDN, KDA, Layer


def _pairs(b):
    return list(zip(b.excess, b.deficit))


def test_hand_worked_even_split():
    # N = 20, P = 4: q = 5, m = 0, every target 5.  Rank 0 keeps 5 of 10,
    # rank 2 keeps 5 of 7; rank 1 has room at positions 3, 4, rank 3 at 0..4.
    b = oracle.storage_balance([10, 3, 7, 0], 4)
    assert b.t == [5, 5, 5, 5] and b.keep == [5, 3, 5, 0] and b.slot_units == 5
    assert _pairs(b) == [((0, 5), (1, 3)), ((0, 6), (1, 4)), ((0, 7), (3, 0)), ((0, 8), (3, 1)),
                         ((0, 9), (3, 2)), ((2, 5), (3, 3)), ((2, 6), (3, 4))]
    assert b.M_remote == 7
    assert b.send_units().tolist() == [[0, 2, 0, 3], [0, 0, 0, 0], [0, 0, 0, 2], [0, 0, 0, 0]]


def test_hand_worked_remainder_and_tie_order():
    # N = 23, P = 4: q = 5, m = 3.  Sorted by (-n_r, r): ranks 1, 2 (9 each,
    # the lower index first), 0 (4), 3 (1): targets 6, 6, 6 and 5.
    b = oracle.storage_balance([4, 9, 9, 1], 4)
    assert b.t == [6, 6, 6, 5] and b.keep == [4, 6, 6, 1] and b.slot_units == 6
    assert _pairs(b) == [((1, 6), (0, 4)), ((1, 7), (0, 5)), ((1, 8), (3, 1)),
                         ((2, 6), (3, 2)), ((2, 7), (3, 3)), ((2, 8), (3, 4))]
    assert b.M_remote == 6
    # ties broken by rank: ranks 0, 1 and 3 hold 6 units, only rank 0 gets q + 1
    b = oracle.storage_balance([6, 6, 3, 6], 4)
    assert b.t == [6, 5, 5, 5]
    assert _pairs(b) == [((1, 5), (2, 3)), ((3, 5), (2, 4))]
    # already balanced: nothing moves, the all-to-all is skipped
    b = oracle.storage_balance([5, 5, 5, 6], 4)
    assert b.t == [5, 5, 5, 6] and b.M_remote == 0


def test_indivisible_head_forces_remote_traffic():
    # one KDA head with 113 retained channels on rank 0, none on rank 1
    b = oracle.storage_balance([113, 0], 2)
    assert b.t == [57, 56] and b.M_remote == 56 and b.slot_units == 57


def test_moved_units_are_minimal_by_brute_force():
    # Any placement that stores t_r units on every rank must move at least
    # sum_r max(0, n_r - t_r) units; enumerate all placements of tiny cases.
    for P, top in ((2, 4), (3, 2)):
        for n in itertools.product(range(top + 1), repeat=P):
            b = oracle.storage_balance(list(n), P)
            src = [r for r in range(P) for _ in range(n[r])]
            best = None
            for owner in itertools.product(range(P), repeat=len(src)):
                if [owner.count(r) for r in range(P)] != b.t:
                    continue
                moved = sum(o != s for o, s in zip(owner, src))
                best = moved if best is None else min(best, moved)
            assert best == b.M_remote, (n, best, b.M_remote)
            assert b.M_remote == sum(max(0, n[r] - b.t[r]) for r in range(P))


def test_target_invariants_random():
    rng = np.random.default_rng(40)
    for _ in range(200):
        P = int(rng.integers(1, 9))
        n = rng.integers(0, 50, P).tolist()
        b = oracle.storage_balance(n, P)
        N = sum(n)
        assert sum(b.t) == N and max(b.t) - min(b.t) <= 1
        assert b.slot_units == math.ceil(N / P) == max(b.t)
        # the slot width depends on N only (same worst rank for any placement)
        assert oracle.storage_balance(list(rng.permutation(n)), P).slot_units == b.slot_units
        stored = [0] * P
        seen = set()
        for s in range(P):
            for i in range(n[s]):
                d, p = b.dest_of(s, i)
                assert 0 <= p < b.t[d]
                assert (d, p) not in seen
                seen.add((d, p))
                stored[d] += 1
                if n[s] <= b.t[s]:
                    assert d == s and p == i          # a rank at or under target keeps all
        assert stored == b.t
        assert b.send_units().sum() == b.M_remote and np.all(np.diag(b.send_units()) == 0)
        # the q + 1 targets go to the largest ranks
        big = sorted(range(P), key=lambda r: (-n[r], r))[:N % P]
        assert all(b.t[r] == N // P + 1 for r in big)


def _model(kind, H, d, seed, conv=64):
    rng = np.random.default_rng(seed)
    n = H if kind == GDN else H * d
    A = rng.normal(0, 1.5, n) if kind == KDA else rng.uniform(-1, 2, n)
    return Layer(kind, H, d, d, A.astype(np.float32), rng.normal(0, 1, n).astype(np.float32),
                 conv)


def _unique_dense(plan, n, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2 ** 32, (n, plan.dense_bytes // 4), dtype=np.uint32).view(np.uint8)


@pytest.mark.parametrize("kind,P,w_max", [(KDA, 2, 8), (KDA, 4, 12), (GDN, 2, 8), (GDN, 4, 8)])
def test_store_load_round_trip(kind, P, w_max):
    d = 8
    layers = [_model(kind, 8, d, 41 + l, conv=16 * P) for l in range(3)]
    plans = oracle.rank_plans(layers, P, w_max=w_max)
    b = oracle.plans_balance(plans)
    assert b.N == sum(p.B_temp_rag for p in plans) // plans[0].layers[0].unit_bytes
    n_ck = 2
    dense = [_unique_dense(p, n_ck, 50 + r) for r, p in enumerate(plans)]
    pools = [np.zeros((n_ck, oracle.slot_bytes_tp(p, b)), np.uint8) for p in plans]
    sends = [np.zeros((n_ck, max(1, oracle.send_bytes_tp(p, b, r))), np.uint8)
             for r, p in enumerate(plans)]
    for r, p in enumerate(plans):
        oracle.pack_tp(p, b, r, dense[r], [1, 0], pools[r], [0, 1], sends[r], [0, 1])
    for ck in range(n_ck):
        oracle.exchange_store(plans, b, [s[ck] for s in sends], pools, ck)
    # every stored unit sits where the map says: unit i of rank s is the i-th
    # retained unit of its ragged pack
    for s, p in enumerate(plans):
        ub = p.layers[0].unit_bytes
        ragged = np.zeros((1, p.slot_bytes), np.uint8)
        oracle.pack(p, dense[s], [1], ragged, [0])
        for i in range(b.n[s]):
            dd, pos = b.dest_of(s, i)
            assert np.array_equal(pools[dd][0, pos * ub:(pos + 1) * ub], ragged[0, i * ub:(i + 1) * ub])
    # the send row: groups by destination rank (ascending), each in the
    # excess list's order, with the all-to-all split sizes as group sizes
    M = b.send_units()
    for s, p in enumerate(plans):
        ub = p.layers[0].unit_bytes
        ragged = np.zeros((1, p.slot_bytes), np.uint8)
        oracle.pack(p, dense[s], [1], ragged, [0])
        order = [i for d in range(P) for (s2, i), (d2, _) in zip(b.excess, b.deficit)
                 if s2 == s and d2 == d]
        assert len(order) == M[s].sum()
        for j, i in enumerate(order):
            assert np.array_equal(sends[s][0, j * ub:(j + 1) * ub], ragged[0, i * ub:(i + 1) * ub])
    # load back into fresh compute-local states
    recvs = [np.zeros_like(s) for s in sends]
    for ck in range(n_ck):
        oracle.exchange_load(plans, b, pools, ck, [rv[ck] for rv in recvs])
    for r, p in enumerate(plans):
        out = np.full_like(dense[r], 0xAB)
        oracle.unpack_tp(p, b, r, pools[r], [0, 1], recvs[r], [0, 1], out, [1, 0])
        exp = np.full_like(dense[r], 0xAB)
        ragged = np.zeros((n_ck, p.slot_bytes), np.uint8)
        oracle.pack(p, dense[r], [0, 1], ragged, [0, 1])
        oracle.unpack_zero_fill(p, ragged, [0, 1], exp, [0, 1])
        assert np.array_equal(out, exp), f"rank {r}"
    if b.M_remote:
        assert any(oracle.send_bytes_tp(p, b, r) > 0 for r, p in enumerate(plans))


def test_tp1_is_the_plain_ragged_slot():
    layers = [_model(KDA, 4, 8, 60 + l) for l in range(2)]
    (p,) = oracle.rank_plans(layers, 1, w_max=8)
    b = oracle.plans_balance([p])
    assert b.M_remote == 0 and b.slot_units * p.layers[0].unit_bytes == p.B_temp_rag
    dense = _unique_dense(p, 1, 61)
    a = np.zeros((1, oracle.slot_bytes_tp(p, b)), np.uint8)
    oracle.pack_tp(p, b, 0, dense, [0], a, [0], np.zeros((1, 1), np.uint8), [0])
    ref = np.zeros((1, p.slot_bytes), np.uint8)
    oracle.pack(p, dense, [0], ref, [0])
    assert np.array_equal(a, ref)


def test_rank_layers_split_heads_and_parameters():
    lay = _model(KDA, 8, 4, 70, conv=32)
    parts = oracle.rank_layers([lay], 4, 2)
    assert parts[0].n_heads == 2 and parts[0].conv_bytes == 8
    assert np.array_equal(parts[0].A_log, lay.A_log[16:24])
    g = _model(GDN, 8, 4, 71, conv=32)
    assert np.array_equal(oracle.rank_layers([g], 4, 3)[0].dt_bias, g.dt_bias[6:8])
