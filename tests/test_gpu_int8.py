"""GPU parity of the INT8 checkpoint pack and zero-fill unpack ([dasc]
Appendix E.1 Eq. 10) against the fp32 oracle, bit-exact, through the C ABI:
full-size workloads (sampled checkpoints against the oracle, every checkpoint
against the zero-fill and conv properties), odd shapes, non-finite states
and the unsupported-shape error."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import log, mask_words

pytestmark = pytest.mark.gpu

R = pytest.importorskip("recurrent_state_cache_amd")


def _plans(cfg):
    return (R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max).upload(),
            oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max))


def _run(P, O, dense, n, sample, seed):
    lo = oracle.Int8Layout(O)
    assert P.info()["int8_slot_bytes"] == lo.slot_bytes
    dev = dense.device
    src = np.random.default_rng(seed).permutation(n).astype(np.int32)
    dst = np.random.default_rng(seed + 1).permutation(n).astype(np.int32)
    pool = torch.full((n, lo.slot_bytes), 0xAB, dtype=torch.uint8, device=dev)
    R.ckpt_pack_int8(P, dense, torch.from_numpy(src).to(dev), pool, torch.from_numpy(dst).to(dev))
    torch.cuda.synchronize()
    assert P.status() == 0
    db = O.dense_bytes
    for i in sample:
        host = dense[int(src[i]), :db].cpu().numpy()[None].copy()
        exp = np.full((1, lo.slot_bytes), 0xAB, np.uint8)
        oracle.pack_int8(O, host, [0], exp, [0])
        got = pool[int(dst[i])].cpu().numpy()
        # padding bytes between the blocks are never written
        assert np.array_equal(got, exp[0]), f"pack_int8 mismatch at entry {i}"
    out = torch.full((n, db), 0xFF, dtype=torch.uint8, device=dev)
    R.ckpt_unpack_int8_zero_fill(P, pool, torch.from_numpy(dst).to(dev), out,
                                 torch.from_numpy(src).to(dev))
    torch.cuda.synchronize()
    assert P.status() == 0
    # every checkpoint: local units +0.0 and conv bytes raw; retained units finite-close
    keep = torch.from_numpy(mask_words(O).view(np.int32)).to(dev)
    conv0 = O.B_temp_dense
    for j in range(n):
        o = out[j].view(torch.int32)
        assert bool(((o & ~keep) == 0).all()), f"unpack_int8: local units of checkpoint {j}"
        assert torch.equal(out[j, conv0:], dense[j, conv0:db]), f"unpack_int8: conv of {j}"
    for i in sample:
        exp = np.full((1, db), 0xFF, np.uint8)
        oracle.unpack_int8_zero_fill(O, pool[int(dst[i])].cpu().numpy()[None].copy(), [0], exp, [0])
        assert np.array_equal(out[int(src[i])].cpu().numpy(), exp[0]), f"unpack_int8 entry {i}"
    return pool, out


@pytest.mark.parametrize("name,n_sample", [("tiny_kda", 2), ("gdn", 2), ("kda", 2), ("mixed", 3)])
def test_int8_full_size(name, n_sample):
    cfg = W.CONFIGS[name]()
    P, O = _plans(cfg)
    n = cfg.n_ckpt
    log(f"[int8] {name}: {n} checkpoints, C_ckpt int8 {P.info()['c_ckpt_int8']:.3f}")
    dense = W.dense_states(cfg, n, device="cuda")
    sample = sorted(set([0, n - 1] + list(np.random.default_rng(4).choice(n, n_sample, replace=False))))
    _run(P, O, dense, n, sample, seed=13)


def _odd_int8_layers(seed):
    rng = np.random.default_rng(seed)
    f = np.float32

    def lay(kind, H, dk, dv, conv):
        n = H * dk if kind == W.KDA else H
        A = rng.uniform(-1, 2, n) if kind == W.GDN else rng.normal(0, 1.5, n)
        return W.Layer(kind, H, dk, dv, A.astype(f), rng.normal(0, 1, n).astype(f), conv)

    return [lay(W.GDN, 6, 8, 8, 32), lay(W.KDA, 3, 8, 4, 48), lay(W.KDA, 2, 16, 16, 0),
            lay(W.GDN, 4, 4, 8, 16), lay(W.KDA, 2, 128, 128, 64), lay(W.GDN, 3, 12, 20, 0),
            lay(W.KDA, 1, 36, 100, 16)]


@pytest.mark.parametrize("w_max", [0, 3, 8, 1 << 30])
def test_int8_odd_shapes(w_max):
    cfg = W.Config("odd8", _odd_int8_layers(5), w_max=w_max)
    P, O = _plans(cfg)
    n = 4
    dense = W.dense_states(cfg, n, device="cuda", seed=w_max % 1000 + 1)
    _run(P, O, dense, n, list(range(n)), seed=w_max % 1000)


def test_int8_non_finite_and_extreme_states():
    cfg = W.Config("odd8", _odd_int8_layers(6), w_max=3)
    P, O = _plans(cfg)
    n = 3
    rng = np.random.default_rng(2)
    host = np.zeros((n, O.dense_bytes), np.uint8)
    vals = rng.standard_normal((n, O.B_temp_dense // 4)).astype(np.float32)
    vals *= np.float32(10.0) ** rng.integers(-30, 30, vals.shape).astype(np.float32)
    special = np.array([np.nan, np.inf, -np.inf, -0.0, 1e-40, -1e-45, 3e38, 1e-9], np.float32)
    pos = rng.choice(vals.size, 400, replace=False)
    vals.reshape(-1)[pos] = special[np.arange(400) % len(special)]
    host[:, :O.B_temp_dense] = vals.view(np.uint8)
    host[:, O.B_temp_dense:] = rng.integers(0, 256, (n, O.B_conv), dtype=np.uint8)
    dense = torch.from_numpy(host).cuda()
    _run(P, O, dense, n, list(range(n)), seed=3)


def test_int8_error_bound_against_the_state():
    # independent of the oracle: every retained entry within half a step
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    dense = W.dense_states(cfg, 2, device="cuda", seed=17)
    lo = oracle.Int8Layout(O)
    pool = torch.zeros((2, lo.slot_bytes), dtype=torch.uint8, device="cuda")
    idx = torch.arange(2, dtype=torch.int32, device="cuda")
    R.ckpt_pack_int8(P, dense, idx, pool, idx)
    out = torch.empty_like(dense)
    R.ckpt_unpack_int8_zero_fill(P, pool, idx, out, idx)
    torch.cuda.synchronize()
    L = O.layers[0]
    S = dense[:, :O.B_temp_dense].view(torch.float32).reshape(2, L.n_heads, L.d_v, L.d_k).cpu()
    Sh = out[:, :O.B_temp_dense].view(torch.float32).reshape(2, L.n_heads, L.d_v, L.d_k).cpu()
    keep = torch.from_numpy(L.retained.reshape(L.n_heads, 1, L.d_k)).expand(2, -1, L.d_v, -1)
    step = S.abs().amax(dim=2, keepdim=True).clamp_min(1e-8) / 127
    err = (Sh - S).abs()
    assert bool((err[keep] <= (step * (0.5 + 1e-5)).expand_as(S)[keep]).all())
    assert bool((Sh[~keep] == 0).all())


def _tie_states(O, n, seed):
    """Dense states whose quotients S / s sit on and next to half-integers:
    each retained column's first row is +-127 s (so the column maximum gives
    s back), the others (k + 1/2 + delta) s in fp32 for deltas from 0 up to
    1e-4 (exact ties, one-ulp neighbours and values just inside and outside
    a few 1e-5 of the tie)."""
    rng = np.random.default_rng(seed)
    f = np.float32
    deltas = np.array([0, 0, 0, 1e-7, -1e-7, 1e-6, -1e-6, 2e-5, -2e-5, 5e-5, -5e-5, 7e-5,
                       -7e-5, 1e-4, -1e-4], np.float64)
    host = np.zeros((n, O.dense_bytes), np.uint8)
    for c in range(n):
        off = 0
        parts = []
        for L in O.layers:
            H, dv, dk = L.n_heads, L.d_v, L.d_k
            s = (f(2.0) ** rng.integers(-20, 20, (H, 1, dk))).astype(f) * \
                rng.uniform(1, 2, (H, 1, dk)).astype(f)
            k = rng.integers(-127, 127, (H, dv, dk)).astype(np.float64)
            d = deltas[rng.integers(0, len(deltas), (H, dv, dk))]
            S = ((k + 0.5 + d) * s.astype(np.float64)).astype(f)
            if dv > 1:
                S[:, 0, :] = (f(127.0) * s[:, 0, :]) * np.where(rng.random((H, dk)) < 0.5, f(-1), f(1))
            parts.append(S.reshape(-1))
        t = np.concatenate(parts)
        host[c, :t.nbytes] = t.view(np.uint8)
        host[c, O.B_temp_dense:] = rng.integers(0, 256, O.B_conv, dtype=np.uint8)
    return host


def test_int8_rounding_ties_and_near_ties():
    # exercises the exact-division route of the pack on most blocks
    cfg = W.Config("odd8", _odd_int8_layers(8), w_max=3)
    P, O = _plans(cfg)
    n = 3
    dense = torch.from_numpy(_tie_states(O, n, seed=21)).cuda()
    _run(P, O, dense, n, list(range(n)), seed=5)


def test_int8_rejects_unsupported_widths():
    lay = W.Layer(W.GDN, 2, 128, 160, np.full(2, -8.0, np.float32), np.zeros(2, np.float32), 0)
    cfg = W.Config("wide", [lay], w_max=4)
    P, O = _plans(cfg)
    dense = torch.zeros((1, O.dense_bytes), dtype=torch.uint8, device="cuda")
    pool = torch.zeros((1, max(P.info()["int8_slot_bytes"], 16)), dtype=torch.uint8, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(R.DascError) as e:
        R.ckpt_pack_int8(P, dense, idx, pool, idx)
    assert e.value.code == -5


def test_int8_kda_column_blocks_full_empty_and_edges():
    # d = 128 KDA heads pack as four 32-channel column blocks in one
    # workgroup (the INT8 pack list then holds only such heads and copies);
    # full, empty, sparse and edge blocks
    from helpers import block_pattern_layers
    cfg = W.Config("blocks", block_pattern_layers(), w_max=64)
    P, O = _plans(cfg)
    n = 3
    dense = W.dense_states(cfg, n, device="cuda", seed=23)
    _run(P, O, dense, n, list(range(n)), seed=23)
    # raw random bits: NaN, infinite and denormal entries inside the blocks
    g = torch.Generator(device="cuda")
    g.manual_seed(29)
    dense = torch.randint(0, 256, (n, O.dense_bytes), dtype=torch.uint8, device="cuda", generator=g)
    _run(P, O, dense, n, list(range(n)), seed=29)


@pytest.mark.parametrize("unaligned", [False, True])
def test_int8_block_heads_beside_whole_heads(unaligned):
    # d = 128 heads pack as four 32-column blocks in one workgroup, other
    # heads whole: GDN layers of 5 and 11 heads with a few retained, a KDA
    # layer whose blocks are full, empty or sparse, a d = 64 GDN layer in
    # between (so one list holds both kinds of piece), and conv bytes;
    # bit-exact.  unaligned: a KDA layer of d_v = 4 with 3 retained channels
    # in front leaves every later INT8 payload offset at 12 mod 16 (the
    # block heads then store 4-byte words).
    f = np.float32
    z = lambda n: np.zeros(n, f)
    g5 = np.array([-4.0, 1.0, -4.0, -4.0, 1.0], f)        # heads 0, 2, 3 retained at W_max 64
    g11 = np.where(np.arange(11) % 3 == 0, -4.0, 1.0).astype(f)
    keep = np.zeros((3, 128), bool)
    keep[0, :40] = True
    keep[1, [5, 127]] = True
    kd = np.where(keep, -4.0, 1.0).reshape(-1).astype(f)
    layers = [W.Layer(W.GDN, 5, 128, 128, g5, z(5), 32),
              W.Layer(W.KDA, 3, 128, 128, kd, z(384), 0),
              W.Layer(W.GDN, 4, 64, 64, np.array([-4.0, -4.0, 1.0, -4.0], f), z(4), 16),
              W.Layer(W.GDN, 11, 128, 128, g11, z(11), 48)]
    if unaligned:
        k8 = np.array([-4.0, -4.0, -4.0, 1.0, 1.0, 1.0, 1.0, 1.0], f)
        layers = [W.Layer(W.KDA, 1, 8, 4, k8, z(8), 16)] + layers
    cfg = W.Config("block_and_whole", layers, w_max=64, seed=77)
    P, O = _plans(cfg)
    kept = [int(L.retained.sum()) for L in O.layers]
    assert kept == ([3] if unaligned else []) + [3, 42, 3, 4]
    offs = [P.layer(l)["int8_pool_offset"] % 16 for l in range(len(layers))]
    assert offs == ([0, 12, 12, 12, 12] if unaligned else [0, 0, 0, 0])
    n = 5
    dense = W.dense_states(cfg, n, device="cuda")
    _run(P, O, dense, n, list(range(n)), seed=21)
