"""The benchmark's work accounting for the refresh with per-head Eq. 7
windows, recounted from the oracle plan: head-token replays (each replayed
head (l, h) of request r replays min(W_lh, n_r) tokens), flops (5 d_v d_k
per replay) and algorithmic HBM bytes (the replayed tokens' k, v, decays
and beta, plus the write-back of every 32-channel row segment that holds a
local column); and the CPU baseline's layer-pair sample."""
import os
import sys

import numpy as np
import pytest

import oracle
import workloads as W

R = pytest.importorskip("recurrent_state_cache_amd")
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.mark.parametrize("name", ["tiny_kda", "widths"])
def test_windowed_work_and_bytes_recounted_from_the_oracle(name):
    if name == "tiny_kda":
        cfg = W.tiny_kda()
    else:
        rng = np.random.default_rng(31)
        f = np.float32
        cfg = W.Config("widths", [
            W.Layer(W.KDA, 2, 32, 32, rng.normal(0, 1.5, 64).astype(f), rng.normal(0, 1, 64).astype(f), 0),
            W.Layer(W.GDN, 6, 16, 16, rng.uniform(-1, 2, 6).astype(f), rng.normal(0, 1, 6).astype(f), 16),
        ], w_max=16)
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    O = oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    Wn = np.array([0, 3, 9, 40])
    # sectors (8 channels of a row) of a replayed KDA head holding both a
    # local and a retained channel, read once per row and request
    reads = 0
    for li, L in enumerate(O.layers):
        if L.kind != oracle.KDA:
            continue
        for h in O.refreshed_heads(li):
            loc = ~L.retained.reshape(L.n_heads, L.d_k)[h]
            mixed = sum(1 for c0 in range(0, L.d_k, 8)
                        if loc[c0:c0 + 8].any() and not loc[c0:c0 + 8].all())
            reads += mixed * 32 * L.d_v * len(Wn)
    assert bench._windowed_sector_reads(P, Wn) == reads
    for decay_bytes in (2, 4):
        ht = flops = nbytes = 0
        for li, L in enumerate(O.layers):
            kda = L.kind == oracle.KDA
            for h in O.refreshed_heads(li):
                w = O.head_window(li, int(h))
                if kda:
                    loc = ~L.retained.reshape(L.n_heads, L.d_k)[h]
                    # channels of the 32-channel row segments holding a local column
                    cols = sum(min(32, L.d_k - c0) for c0 in range(0, L.d_k, 32)
                               if loc[c0:c0 + 32].any())
                else:
                    cols = L.d_k
                for n_r in Wn:
                    t = min(w, int(n_r))
                    ht += t
                    flops += 5 * L.d_v * L.d_k * t
                    nbytes += t * (2 * L.d_k + 2 * L.d_v + (L.d_k if kda else 1) * decay_bytes + 4)
                    nbytes += cols * L.d_v * 4
        assert bench._windowed_work(P, Wn) == (flops, ht)
        assert bench._windowed_bytes(P, Wn, decay_bytes=decay_bytes) == nbytes
        assert ht > 0


def test_mover_bytes_recounted_from_the_oracle():
    """pack reads every retained GDN head and, of a d = 128 KDA head, each
    32-channel block with a retained channel (whole heads at other widths),
    writes the ragged payload and copies conv; unpack reads the payload and
    conv and writes the dense checkpoint; INT8 pack reads as pack does."""
    from helpers import block_pattern_layers
    rng = np.random.default_rng(5)
    f = np.float32
    layers = block_pattern_layers() + [
        W.Layer(W.KDA, 3, 32, 32, rng.normal(-1, 2, 96).astype(f), np.zeros(96, f), 32),
        W.Layer(W.GDN, 5, 16, 16, rng.uniform(-3, 2, 5).astype(f), np.zeros(5, f), 16)]
    cfg = W.Config("movers", layers, w_max=64)
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    O = oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    read = read_q = 0
    for L in O.layers:
        if L.kind == oracle.GDN:
            read += int(L.retained.sum()) * L.d_v * L.d_k * 4
            read_q += int(L.retained.sum()) * L.d_v * L.d_k * 4
            continue
        heads = L.retained.reshape(L.n_heads, L.d_k)
        if L.d_k == 128 and L.d_v == 128:
            for h in range(L.n_heads):
                for b in range(4):
                    read += 128 * 32 * 4 if heads[h, 32 * b:32 * (b + 1)].any() else 0
        else:
            read += int(heads.any(axis=1).sum()) * L.d_v * L.d_k * 4
    read_q = read
    # the pattern has empty blocks in heads that are read
    assert read < sum(int(L.retained.reshape(L.n_heads, -1).any(axis=1).sum()) * L.d_v * L.d_k * 4
                      for L in O.layers)
    q = sum(int(L.retained.sum()) * (L.d_v * L.d_k if L.kind == oracle.GDN else L.d_v) for L in O.layers)
    q += sum(int(L.retained.sum()) * (L.d_k if L.kind == oracle.GDN else 1) * 4 for L in O.layers)
    pack, unpack, pack_q, unpack_q = bench._algorithmic_bytes(P)
    assert pack == read + O.B_temp_rag + 2 * O.B_conv
    assert unpack == O.B_temp_rag + O.B_temp_dense + 2 * O.B_conv
    assert pack_q == read_q + q + 2 * O.B_conv
    assert unpack_q == q + O.B_temp_dense + 2 * O.B_conv


def test_cpu_sample_layer_pairs_replay_the_full_plans_heads():
    # The CPU baseline replays a pair of layers with a plan of those layers
    # only: a unit's retention depends on its own parameters, so the pair
    # plan replays exactly the heads (and windows) the full plan does.
    cfg = W.mixed(n_ckpt=2, n_req=2)
    O = oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    for j in (0, 5, 12):
        sub = oracle.build_plan(cfg.layers[2 * j:2 * j + 2], cfg.a_s, cfg.eps, cfg.w_max)
        for i in range(2):
            heads = O.refreshed_heads(2 * j + i)
            assert np.array_equal(sub.refreshed_heads(i), heads)
            assert [sub.head_window(i, int(h)) for h in heads] == \
                [O.head_window(2 * j + i, int(h)) for h in heads]
