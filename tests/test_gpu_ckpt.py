"""GPU parity of pack and zero-fill unpack against the oracle (bit-exact),
through the C ABI, at the benchmark's full sizes (sampled checkpoints against
the oracle, every checkpoint against the mask property) and on small odd
shapes, special bit patterns and error paths."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import block_pattern_layers, log, mask_words

pytestmark = pytest.mark.gpu

R = pytest.importorskip("recurrent_state_cache_amd")


def _plans(cfg):
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max).upload()
    O = oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    return P, O


def _perm(n, seed):
    return np.random.default_rng(seed).permutation(n).astype(np.int32)


def _run_and_check(cfg, P, O, dense, n, sample, seed, pool_pad=0, dense_pad=0):
    dev = dense.device
    src = _perm(n, seed)
    dst = _perm(n, seed + 1)
    slot = O.slot_bytes
    pool_full = torch.full((n, slot + pool_pad), 0xAB, dtype=torch.uint8, device=dev)
    pool = pool_full[:, :slot]                 # rows may be padded
    R.ckpt_pack(P, dense, torch.from_numpy(src).to(dev), pool, torch.from_numpy(dst).to(dev))
    torch.cuda.synchronize()
    assert P.status() == 0
    db = O.dense_bytes
    for i in sample:
        host = dense[int(src[i])].cpu().numpy()[None, :db].copy()
        exp = np.zeros((1, slot), np.uint8)
        oracle.pack(O, host, [0], exp, [0])
        got = pool_full[int(dst[i]), :slot].cpu().numpy()
        assert np.array_equal(got, exp[0]), f"pack mismatch at entry {i}"
    if pool_pad:
        assert bool((pool_full[:, slot:] == 0xAB).all()), "pack wrote into row padding"
    # unpack slot dst[i] into checkpoint src[i] of a fresh buffer
    out_full = torch.full((n, db + dense_pad), 0xFF, dtype=torch.uint8, device=dev)
    out = out_full[:, :db]
    R.ckpt_unpack_zero_fill(P, pool, torch.from_numpy(dst).to(dev), out,
                            torch.from_numpy(src).to(dev))
    torch.cuda.synchronize()
    assert P.status() == 0
    mask = torch.from_numpy(mask_words(O).view(np.int32)).to(dev)
    for j in range(n):
        d = dense[j, :db].view(torch.int32)
        assert torch.equal(out_full[j, :db].view(torch.int32), d & mask), f"round trip {j}"
    for i in sample:
        exp = np.full((1, db), 0xFF, np.uint8)
        oracle.unpack_zero_fill(O, pool_full[int(dst[i]), :slot].cpu().numpy()[None].copy(), [0],
                                exp, [0])
        assert np.array_equal(out_full[int(src[i]), :db].cpu().numpy(), exp[0]), f"unpack {i}"
    if dense_pad:
        assert bool((out_full[:, db:] == 0xFF).all()), "unpack wrote into row padding"
    return pool_full, out_full


@pytest.mark.parametrize("name,n_sample", [("tiny_kda", 2), ("gdn", 3), ("kda", 3), ("mixed", 30)])
def test_pack_unpack_full_size(name, n_sample):
    cfg = W.CONFIGS[name]()
    log(f"[ckpt] {name}: {cfg.n_ckpt} checkpoints, W_max={cfg.w_max}")
    P, O = _plans(cfg)
    n = cfg.n_ckpt
    dense = W.dense_states(cfg, n, device="cuda")
    sample = sorted(set([0, n - 1] + list(np.random.default_rng(7).choice(n, n_sample, replace=False))))
    _run_and_check(cfg, P, O, dense, n, sample, seed=11)


def _odd_layers(seed):
    rng = np.random.default_rng(seed)
    f = np.float32
    return [
        W.Layer(W.GDN, 6, 8, 8, rng.uniform(-1, 2, 6).astype(f), rng.normal(0, 1, 6).astype(f), 32),
        W.Layer(W.KDA, 3, 8, 4, rng.normal(0, 1.5, 24).astype(f), rng.normal(0, 1, 24).astype(f), 48),
        W.Layer(W.KDA, 2, 16, 16, rng.normal(0, 1.5, 32).astype(f), rng.normal(0, 1, 32).astype(f), 0),
        W.Layer(W.GDN, 4, 4, 8, rng.uniform(-1, 2, 4).astype(f), rng.normal(0, 1, 4).astype(f), 16),
        W.Layer(W.KDA, 2, 128, 128, rng.normal(0, 1.5, 256).astype(f), rng.normal(0, 1, 256).astype(f), 64),
        W.Layer(W.GDN, 3, 128, 160, rng.uniform(-1, 2, 3).astype(f), rng.normal(0, 1, 3).astype(f), 0),
    ]


@pytest.mark.parametrize("w_max", [0, 2, 8, 64, 1 << 30])
def test_odd_shapes_random_bits(w_max):
    # random bytes cover every fp32 bit pattern class: NaN payloads, -0.0,
    # denormals, infinities.
    layers = _odd_layers(3)
    cfg = W.Config("odd", layers, w_max=w_max)
    P, O = _plans(cfg)
    n = 5
    g = torch.Generator(device="cuda")
    g.manual_seed(w_max % 1000)
    dense = torch.randint(0, 256, (n, O.dense_bytes), dtype=torch.uint8, device="cuda", generator=g)
    _run_and_check(cfg, P, O, dense, n, list(range(n)), seed=w_max % 1000)


def test_padded_row_strides():
    cfg = W.Config("odd", _odd_layers(4), w_max=8)
    P, O = _plans(cfg)
    n = 4
    dense_full = torch.randint(0, 256, (n, O.dense_bytes + 48), dtype=torch.uint8, device="cuda")
    dense = dense_full[:, :O.dense_bytes]
    _run_and_check(cfg, P, O, dense, n, list(range(n)), seed=5, pool_pad=32, dense_pad=16)


def test_special_values_survive():
    cfg = W.tiny_kda()
    cfg.w_max = 0                     # retain everything: pack is a full copy
    P, O = _plans(cfg)
    sv = W.special_values_f32()
    host = np.resize(sv, O.dense_bytes // 4).view(np.uint8)[None].repeat(2, 0)
    dense = torch.from_numpy(host.copy()).cuda()
    _run_and_check(cfg, P, O, dense, 2, [0, 1], seed=9)


def test_zero_entries_is_a_no_op():
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    dense = W.dense_states(cfg, 2, device="cuda")
    pool = torch.full((2, O.slot_bytes), 7, dtype=torch.uint8, device="cuda")
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    R.ckpt_pack(P, dense, e, pool, e)
    R.ckpt_unpack_zero_fill(P, pool, e, dense, e)
    torch.cuda.synchronize()
    assert bool((pool == 7).all())


def test_out_of_range_index_is_skipped_and_flagged():
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    dense = W.dense_states(cfg, 2, device="cuda")
    pool = torch.full((3, O.slot_bytes), 7, dtype=torch.uint8, device="cuda")
    src = torch.tensor([0, 2, -1], dtype=torch.int32, device="cuda")   # 2 and -1 are bad
    dst = torch.tensor([1, 0, 2], dtype=torch.int32, device="cuda")
    R.ckpt_pack(P, dense, src, pool, dst)
    torch.cuda.synchronize()
    assert P.status() & R.STATUS_BAD_INDEX
    assert P.status() == 0                          # cleared by the first read
    assert bool((pool[0] == 7).all()) and bool((pool[2] == 7).all())
    exp = np.zeros((1, O.slot_bytes), np.uint8)
    oracle.pack(O, dense[0].cpu().numpy()[None].copy(), [0], exp, [0])
    assert np.array_equal(pool[1].cpu().numpy(), exp[0])


def test_host_validation_on_device_buffers():
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    dense = W.dense_states(cfg, 2, device="cuda")
    pool = torch.zeros((2, O.slot_bytes), dtype=torch.uint8, device="cuda")
    idx = torch.arange(2, dtype=torch.int32, device="cuda")
    bad = dense.view(-1)[:2 * (O.dense_bytes - 16)].view(2, O.dense_bytes - 16)
    with pytest.raises(R.DascError) as e:
        R.ckpt_pack(P, bad, idx, pool, idx)              # stride below dense_bytes
    assert e.value.code == -1
    with pytest.raises(R.DascError):
        R.ckpt_pack(P, dense, idx, dense.view(2, -1)[:, :O.slot_bytes], idx)  # overlap
    with pytest.raises(TypeError):
        R.ckpt_pack(P, dense, idx.long(), pool, idx)


def test_kda_column_blocks_full_empty_and_edges():
    cfg = W.Config("blocks", block_pattern_layers(), w_max=64)
    P, O = _plans(cfg)
    kept = O.layers[0].retained.reshape(4, 128)
    assert kept[0, :32].all() and not kept[0, 32:64].any() and kept[0, 127]
    assert not kept[3].any() and kept[2].sum() == 126
    n = 3
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    dense = torch.randint(0, 256, (n, O.dense_bytes), dtype=torch.uint8, device="cuda", generator=g)
    _run_and_check(cfg, P, O, dense, n, list(range(n)), seed=17)
