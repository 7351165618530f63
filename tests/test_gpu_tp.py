"""GPU parity of the TP storage-balancing store and load ([dasc] §4.3,
Appendix B.1(b)) against the oracle, bit-exact, through the C ABI: every
rank's pack / partition (slot rows and send rows), the stored slots after
the exchange, and every rank's zero-fill load after the inverse exchange.
One GPU holds all tp ranks' buffers; the all-to-all between them is done
here with device copies that follow the library's split matrix."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import log

pytestmark = pytest.mark.gpu

R = pytest.importorskip("recurrent_state_cache_amd")


def _exchange_store(M, keep, ub, sends, pools, send_rows, slot_rows):
    tp = len(keep)
    for d in range(tp):
        pos = int(keep[d])
        for s in range(tp):
            c = int(M[s, d])
            if c:
                off = int(M[s, :d].sum())
                pools[d][slot_rows, pos * ub:(pos + c) * ub] = \
                    sends[s][send_rows, off * ub:(off + c) * ub]
                pos += c


def _exchange_load(M, keep, ub, pools, recvs, slot_rows, recv_rows):
    tp = len(keep)
    for d in range(tp):
        pos = int(keep[d])
        for s in range(tp):
            c = int(M[s, d])
            if c:
                off = int(M[s, :d].sum())
                recvs[s][recv_rows, off * ub:(off + c) * ub] = \
                    pools[d][slot_rows, pos * ub:(pos + c) * ub]
                pos += c


def _round_trip(layers, a_s, eps, w_max, tp, n_ck, label, sample=None, seed=0):
    orac = oracle.rank_plans(layers, tp, a_s, eps, w_max)
    b = oracle.plans_balance(orac)
    plans = [R.Plan(layers, a_s, eps, w_max, tp=tp, rank=r).upload() for r in range(tp)]
    M, n, t = plans[0].tp_splits()
    infos = [p.tp_info() for p in plans]
    keep = [i["keep"] for i in infos]
    ub = infos[0]["unit_bytes"]
    log(f"[tp] {label}: tp {tp}, n_r {n.tolist()}, t_r {t.tolist()}, M_remote "
        f"{infos[0]['m_remote']}, slot units {infos[0]['slot_units']}")
    assert infos[0]["m_remote"] == b.M_remote
    rng = np.random.default_rng(seed)
    src, slot, sidx = (torch.from_numpy(rng.permutation(n_ck).astype(np.int32)).cuda()
                       for _ in range(3))
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    dense = [torch.randint(0, 256, (n_ck, p.info()["dense_bytes"]), generator=g,
                           dtype=torch.uint8, device="cuda") for p in plans]
    pools = [torch.full((n_ck, i["slot_bytes"]), 0xAB, dtype=torch.uint8, device="cuda")
             for i in infos]
    sends = [torch.full((n_ck, max(16, i["send_bytes"])), 0xCD, dtype=torch.uint8,
                        device="cuda") for i in infos]
    for r, p in enumerate(plans):
        R.ckpt_pack_tp(p, dense[r], src, pools[r], slot, sends[r], sidx)
    torch.cuda.synchronize()
    assert all(p.status() == 0 for p in plans)

    # oracle: pack / partition of every rank on the sampled checkpoints
    ck = range(n_ck) if sample is None else sample
    src_h, slot_h, sidx_h = (x.cpu().numpy() for x in (src, slot, sidx))
    o_pools = [np.full((n_ck, i["slot_bytes"]), 0xAB, np.uint8) for i in infos]
    o_sends = [np.full((n_ck, max(16, oracle.send_bytes_tp(O, b, r))), 0xCD, np.uint8)
               for r, O in enumerate(orac)]
    for r, O in enumerate(orac):
        host = dense[r].cpu().numpy()
        for i in ck:
            oracle.pack_tp(O, b, r, host, [src_h[i]], o_pools[r], [slot_h[i]], o_sends[r],
                           [sidx_h[i]])
        for i in ck:
            assert np.array_equal(pools[r][slot_h[i]].cpu().numpy(), o_pools[r][slot_h[i]]), \
                f"{label}: rank {r} slot row of entry {i}"
            assert np.array_equal(sends[r][sidx_h[i]].cpu().numpy(), o_sends[r][sidx_h[i]]), \
                f"{label}: rank {r} send row of entry {i}"

    # the exchange, then the stored slots against the oracle's exchange
    _exchange_store(M, keep, ub, sends, pools, sidx.long(), slot.long())
    torch.cuda.synchronize()
    for i in ck:
        oracle.exchange_store(orac, b, [s[sidx_h[i]] for s in o_sends], o_pools, slot_h[i])
    for r in range(tp):
        for i in ck:
            assert np.array_equal(pools[r][slot_h[i]].cpu().numpy(), o_pools[r][slot_h[i]]), \
                f"{label}: stored slot of rank {r}, entry {i}"

    # load: inverse exchange into receive rows, then every rank's unpack
    ridx = torch.from_numpy(rng.permutation(n_ck).astype(np.int32)).cuda()
    dst = torch.from_numpy(rng.permutation(n_ck).astype(np.int32)).cuda()
    recvs = [torch.full_like(s, 0xEE) for s in sends]
    _exchange_load(M, keep, ub, pools, recvs, slot.long(), ridx.long())
    outs = [torch.full_like(d, 0x77) for d in dense]
    for r, p in enumerate(plans):
        R.ckpt_unpack_tp_zero_fill(p, pools[r], slot, recvs[r], ridx, outs[r], dst)
    torch.cuda.synchronize()
    assert all(p.status() == 0 for p in plans)
    ridx_h, dst_h = ridx.cpu().numpy(), dst.cpu().numpy()
    o_recvs = [np.full_like(x, 0xEE) for x in o_sends]
    for i in ck:
        oracle.exchange_load(orac, b, o_pools, slot_h[i], [x[ridx_h[i]] for x in o_recvs])
    for r, O in enumerate(orac):
        host_out = np.full_like(dense[r].cpu().numpy(), 0x77)
        rv = o_recvs[r]
        for i in ck:
            oracle.unpack_tp(O, b, r, o_pools[r], [slot_h[i]], rv, [ridx_h[i]], host_out,
                             [dst_h[i]])
            got = outs[r][dst_h[i]].cpu().numpy()
            assert np.array_equal(got, host_out[dst_h[i]]), f"{label}: load of rank {r}, entry {i}"
            # and the round trip: the rank's own checkpoint, masked
            ragged = np.zeros((1, O.slot_bytes), np.uint8)
            exp = np.zeros((1, O.dense_bytes), np.uint8)
            oracle.pack(O, dense[r].cpu().numpy(), [src_h[i]], ragged, [0])
            oracle.unpack_zero_fill(O, ragged, [0], exp, [0])
            assert np.array_equal(got, exp[0]), f"{label}: round trip of rank {r}, entry {i}"
    return b


def _skewed(kind, H, d, n_layers, seed, conv):
    """Layers whose slow heads cluster on the first ranks (uneven n_r)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_layers):
        n = H if kind == W.GDN else H * d
        head = np.repeat(np.arange(H), 1 if kind == W.GDN else d)
        A = rng.normal(0, 1.0, n) - 2.5 * (head < H // 3) + 1.0 * (head >= H // 2)
        out.append(W.Layer(kind, H, d, d, A.astype(np.float32),
                           rng.normal(0, 1, n).astype(np.float32), conv))
    return out


@pytest.mark.parametrize("tp", [2, 4])
def test_tp_small_kda_skewed(tp):
    layers = _skewed(W.KDA, 8, 16, 3, 80 + tp, conv=64 * tp)
    b = _round_trip(layers, -0.3, 1e-3, 16, tp, 3, f"kda d16 tp{tp}", seed=tp)
    assert b.M_remote > 0


def test_tp_kda_d128_skewed():
    # d = 128: the pack list's 32-channel column blocks, some of whose units
    # straddle the keep boundary into the send row
    layers = _skewed(W.KDA, 4, 128, 2, 71, conv=64)
    b = _round_trip(layers, -0.3, 1e-3, 16, 2, 3, "kda d128 tp2", seed=71)
    assert b.M_remote > 0


@pytest.mark.parametrize("tp", [2, 4])
def test_tp_small_gdn_skewed(tp):
    # 1 KiB units (one copy piece each), some kept, some sent
    layers = _skewed(W.GDN, 8, 16, 4, 90 + tp, conv=32 * tp)
    b = _round_trip(layers, -0.3, 1e-3, 8, tp, 3, f"gdn d16 tp{tp}", seed=10 + tp)
    assert b.M_remote > 0


def test_tp8_kda_full_shape_sampled():
    cfg = W.kda()
    _round_trip(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max, 8, 4, "kda tp8", sample=[0, 3], seed=5)


def test_tp8_gdn_full_shape_sampled():
    cfg = W.gdn()
    _round_trip(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max, 8, 3, "gdn tp8", sample=[1], seed=6)


def test_tp1_equals_plain_pack():
    cfg = W.tiny_kda()
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max).upload()
    dense = W.dense_states(cfg, 2, device="cuda")
    idx = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
    a = torch.zeros((2, P.info()["slot_bytes"]), dtype=torch.uint8, device="cuda")
    c = torch.zeros_like(a)
    R.ckpt_pack(P, dense, idx, a, idx)
    R.ckpt_pack_tp(P, dense, idx, c, idx, None, None)
    out = torch.zeros_like(dense)
    R.ckpt_unpack_tp_zero_fill(P, c, idx, None, None, out, idx)
    ref = torch.zeros_like(dense)
    R.ckpt_unpack_zero_fill(P, a, idx, ref, idx)
    torch.cuda.synchronize()
    assert torch.equal(a, c) and torch.equal(out, ref)
