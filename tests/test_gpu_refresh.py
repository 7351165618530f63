"""GPU parity of the bounded-suffix refresh against the fp64 oracle, through
the C ABI: max error over the written (local) entries, relative to the
Frobenius norm of the fp64 scratch state, must stay within 1e-4; everything
the refresh must not touch (retained units, conv bytes, other checkpoints)
must be bit-identical afterwards."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from helpers import head_state, local_mask_of_head, log, mask_words, refresh_error

pytestmark = pytest.mark.gpu

R = pytest.importorskip("recurrent_state_cache_amd")

TOL = 1e-4


def _plans(cfg):
    return (R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max).upload(),
            oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max))


def _host_rows(x, rows):
    return x[rows[0]:rows[1]].cpu()


def _bits16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _check_requests(P, O, inp, before, after, dst, reqs, layers=None, label="",
                    head_windows=False):
    """Compare the refreshed heads of the given requests (and layers) with
    the oracle; check untouched bytes of those destinations bit-exactly."""
    tok = inp.tok_off.cpu().numpy()
    mask = mask_words(O)
    worst = 0.0
    for r in reqs:
        t0, t1 = int(tok[r]), int(tok[r + 1])
        k = _bits16(_host_rows(inp.k, (t0, t1)))
        v = _bits16(_host_rows(inp.v, (t0, t1)))
        a = _bits16(_host_rows(inp.a, (t0, t1)))
        b = _host_rows(inp.beta, (t0, t1)).numpy()
        ref = oracle.refresh_expected(O, k, v, a, b, np.array([0, t1 - t0]), layers=layers,
                                      head_windows=head_windows)
        d = int(dst[r])
        got = after[d].cpu().numpy()
        old = before[d].cpu().numpy()
        # retained units and conv bytes untouched
        assert np.array_equal(got.view(np.uint32) & mask, old.view(np.uint32) & mask), f"req {r}"
        for (_, li, h), S64 in ref.items():
            local = local_mask_of_head(O, li, h)
            g = head_state(got, O, li, h)
            assert np.all(np.isfinite(g[local]))
            err = refresh_error(g, S64, local)
            worst = max(worst, err)
            assert err <= TOL, f"{label} req {r} layer {li} head {h}: {err:.3e}"
    log(f"[refresh] {label}: worst error {worst:.3e} over requests {list(reqs)}")
    return worst


def test_refresh_tiny_kda_all_heads():
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp = W.refresh_inputs(cfg, Wn, device="cpu")
    inp = W.RefreshInputs(*(x.cuda() for x in (inp.k, inp.v, inp.a, inp.beta, inp.tok_off)))
    dense = W.dense_states(cfg, 3, device="cuda", seed=99)
    before = dense.clone()
    dst = torch.tensor([2, 0], dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    assert torch.equal(dense[1], before[1])                 # not a destination
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), [0, 1], label="tiny")


def test_refresh_kda_full_size_sampled():
    cfg = W.kda_refresh()
    log(f"[refresh] kda: {cfg.n_req} requests x {cfg.window[0]} tokens, "
        f"{len(cfg.layers)} layers x 32 heads")
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    dense = W.dense_states(cfg, cfg.n_req, device="cuda", seed=5)
    before = dense.clone()
    dst = torch.from_numpy(np.random.default_rng(1).permutation(cfg.n_req).astype(np.int32)).cuda()
    R.ckpt_refresh_suffix(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), [0, 37], layers=[0, 19],
                    label="kda")
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), [63], layers=[9], label="kda")


def test_refresh_mixed_sampled():
    cfg = W.mixed(n_ckpt=64)
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    log(f"[refresh] mixed: windows {Wn.min()}..{Wn.max()}, {int(Wn.sum())} tokens")
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    dense = W.dense_states(cfg, cfg.n_req, device="cuda", seed=6)
    before = dense.clone()
    dst = torch.arange(cfg.n_req, dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    reqs = [int(np.argmax(Wn)), int(np.argmin(Wn))]
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), reqs, layers=[0, 1, 26],
                    label="mixed")


def _odd_refresh_layers(seed):
    """Every refresh width (16, 32, 64, 128) as GDN and KDA layers.  The
    GDN layers' one-per-head gate logits shift the KDA layers' gate blocks:
    the d = 32 and d = 128 KDA layers start on a 16-byte boundary (vector
    gate reads), the d = 64 and d = 16 ones do not (element reads)."""
    rng = np.random.default_rng(seed)
    f = np.float32

    def lay(kind, H, d):
        n = H * d if kind == W.KDA else H
        A = rng.uniform(-1, 2, n) if kind == W.GDN else rng.normal(0, 1.5, n)
        return W.Layer(kind, H, d, d, A.astype(f), rng.normal(0, 1, n).astype(f), 0)

    return [lay(W.KDA, 2, 32), lay(W.GDN, 3, 32), lay(W.KDA, 2, 64), lay(W.GDN, 2, 64),
            lay(W.KDA, 1, 16), lay(W.GDN, 3, 16), lay(W.KDA, 2, 128), lay(W.GDN, 8, 16)]


def test_refresh_every_width_and_unaligned_gate_rows():
    cfg = W.Config("widths", _odd_refresh_layers(21), w_max=8, n_req=3, seed=21)
    P, O = _plans(cfg)
    assert P.info()["gate_row"] % 8 == 0
    kda_offsets = [P.layer(l)["gate_row_offset"] for l in range(len(cfg.layers))
                   if cfg.layers[l].kind == W.KDA]
    assert [o % 8 == 0 for o in kda_offsets] == [True, False, False, True], kda_offsets
    for li in range(len(cfg.layers)):
        assert len(O.refreshed_heads(li)) > 0, f"layer {li} replays no head"
    Wn = np.array([5, 16, 37])
    log(f"[refresh] widths 16..128, GDN and KDA, gate offsets {kda_offsets}, windows {list(Wn)}")
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    dense = W.dense_states(cfg, 4, device="cuda", seed=8)
    before = dense.clone()
    dst = torch.tensor([3, 0, 2], dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    assert torch.equal(dense[1], before[1])                 # not a destination
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), [0, 1, 2], label="widths")


def test_zero_window_writes_zero_locals_and_bad_ranges_are_flagged():
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    inp = W.refresh_inputs(cfg, np.array([8, 8]), device="cpu")
    k, v, a, beta = (x.cuda() for x in (inp.k, inp.v, inp.a, inp.beta))
    dense = W.dense_states(cfg, 2, device="cuda", seed=3)
    before = dense.clone()
    tok = torch.tensor([0, 0, 8], dtype=torch.int64, device="cuda")   # request 0 is empty
    dst = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix(P, k, v, a, beta, tok, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    m = torch.from_numpy(mask_words(O).view(np.int32)).cuda()
    assert torch.equal(dense[0].view(torch.int32), before[0].view(torch.int32) & m)
    # a request whose range runs past the tokens is skipped and flagged
    dense2 = before.clone()
    bad = torch.tensor([0, 8, 17], dtype=torch.int64, device="cuda")   # 17 > 16 rows
    R.ckpt_refresh_suffix(P, k, v, a, beta, bad, dense2, dst)
    torch.cuda.synchronize()
    assert P.status() & R.STATUS_BAD_TOKENS
    assert torch.equal(dense2[1], before[1])


def test_recall_invariant_on_gpu():
    # GDN heads that are all local; beta = 1 and keys of exactly unit norm in
    # bf16 (+-1/4 on 16 coordinates): the final state recalls the last value,
    # S_W k_W = v_W, independently of the oracle.
    d, H, T = 128, 4, 40
    lay = W.Layer(W.GDN, H, d, d, np.full(H, 2.0, np.float32), np.zeros(H, np.float32), 0)
    cfg = W.Config("recall", [lay], w_max=64)
    P, O = _plans(cfg)
    assert len(O.refreshed_heads(0)) == H
    rng = np.random.default_rng(8)
    k = np.zeros((T, H, d), np.float32)
    for t in range(T):
        for h in range(H):
            idx = rng.choice(d, 16, replace=False)
            k[t, h, idx] = rng.choice([-0.25, 0.25], 16)
    kt = torch.from_numpy(k.reshape(T, H * d)).to(torch.bfloat16).cuda()
    vt = torch.randn(T, H * d).to(torch.bfloat16).cuda()
    at = torch.randn(T, H).to(torch.bfloat16).cuda()
    bt = torch.ones(T, H, dtype=torch.float32, device="cuda")
    dense = torch.zeros((1, O.dense_bytes), dtype=torch.uint8, device="cuda")
    R.ckpt_refresh_suffix(P, kt, vt, at, bt, torch.tensor([0, T], device="cuda"), dense,
                          torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    row = dense[0].cpu().numpy()
    for h in range(H):
        S = head_state(row, O, 0, h).astype(np.float64)
        vlast = vt[-1, h * d:(h + 1) * d].float().cpu().numpy()
        recall = S @ k[-1, h].astype(np.float64)
        assert np.max(np.abs(recall - vlast)) <= 1e-5 * max(1.0, np.linalg.norm(vlast))


def test_unsupported_refresh_shape_is_rejected():
    lay = W.Layer(W.GDN, 2, 128, 160, np.full(2, 2.0, np.float32), np.zeros(2, np.float32), 0)
    cfg = W.Config("wide", [lay], w_max=64)
    P, _ = _plans(cfg)
    T = 2
    z = torch.zeros(T, 256, dtype=torch.bfloat16, device="cuda")
    dense = torch.zeros((1, P.info()["dense_bytes"]), dtype=torch.uint8, device="cuda")
    with pytest.raises(R.DascError) as e:
        R.ckpt_refresh_suffix(P, z, torch.zeros(T, 320, dtype=torch.bfloat16, device="cuda"),
                              torch.zeros(T, 2, dtype=torch.bfloat16, device="cuda"),
                              torch.zeros(T, 2, device="cuda"),
                              torch.tensor([0, T], device="cuda"), dense,
                              torch.zeros(1, dtype=torch.int32, device="cuda"))
    assert e.value.code == -5


def test_windowed_refresh_every_width():
    # W_max = 64: head windows from 4 to 64, requests shorter and longer
    cfg = W.Config("widths", _odd_refresh_layers(22), w_max=64, n_req=5, seed=22)
    P, O = _plans(cfg)
    wins = sorted({O.head_window(li, int(h)) for li in range(len(cfg.layers))
                   for h in O.refreshed_heads(li)})
    Wn = np.array([0, 3, 17, 70, 130])
    log(f"[refresh] windowed, widths 16..128: head windows {wins}, requests {list(Wn)}")
    assert len(wins) >= 3
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    dense = W.dense_states(cfg, 6, device="cuda", seed=9)
    before = dense.clone()
    dst = torch.tensor([5, 0, 2, 1, 3], dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix_windowed(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    assert torch.equal(dense[4], before[4])                 # not a destination
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), range(5), label="windowed",
                    head_windows=True)


def test_one_chunk_windows_every_width_against_the_oracle():
    # W_max = 16: every head window is at most one chunk, so every launch
    # group (widths 16..128, GDN, KDA with vector and element gate reads)
    # runs the one-chunk kernel; requests shorter than, equal to and longer
    # than the windows
    cfg = W.Config("widths", _odd_refresh_layers(25), w_max=16, n_req=5, seed=25)
    P, O = _plans(cfg)
    wins = sorted({O.head_window(li, int(h)) for li in range(len(cfg.layers))
                   for h in O.refreshed_heads(li)})
    assert max(wins) <= 16 and len(wins) >= 2, wins
    Wn = np.array([0, 5, 16, 40, 3])
    log(f"[refresh] one-chunk windows {wins}, requests {list(Wn)}")
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    dense = W.dense_states(cfg, 5, device="cuda", seed=12)
    before = dense.clone()
    dst = torch.tensor([3, 1, 4, 0, 2], dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix_windowed(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), range(5), label="one-chunk",
                    head_windows=True)


def test_windowed_refresh_kda_and_mixed_sampled():
    for cfg, reqs, layers in ((W.kda_refresh(n_req=8), [0, 7], [0, 19]),
                              (W.mixed(n_ckpt=16, n_req=16), [0, 5], [0, 1, 26])):
        P, O = _plans(cfg)
        Wn = W.windows(cfg)
        wins = sorted({O.head_window(li, int(h)) for li in layers for h in O.refreshed_heads(li)})
        log(f"[refresh] windowed {cfg.name}: W_max {cfg.w_max}, head windows {wins}, "
            f"requests of {Wn.min()}..{Wn.max()} tokens")
        inp = W.refresh_inputs(cfg, Wn, device="cuda")
        dense = W.dense_states(cfg, cfg.n_req, device="cuda", seed=10)
        before = dense.clone()
        dst = torch.arange(cfg.n_req, dtype=torch.int32, device="cuda")
        R.ckpt_refresh_suffix_windowed(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense,
                                       dst)
        torch.cuda.synchronize()
        assert P.status() == 0
        _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), reqs, layers=layers,
                        label=f"windowed {cfg.name}", head_windows=True)


def test_windowed_refresh_keeps_retained_bits():
    # The windowed refresh writes heads that also hold retained channels as
    # whole rows (their retained values read and written back): retained
    # words holding any bit pattern (NaN payloads, infinities, -0.0,
    # denormals, raw random bits) must come back unchanged, and the local
    # entries must still match the oracle.
    cfg = W.kda_refresh(n_req=4)
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(41)
    dense = torch.randint(0, 256, (cfg.n_req, O.dense_bytes), dtype=torch.uint8, device="cuda",
                          generator=g)
    words = dense[:, :O.B_temp_dense].view(torch.int32)
    special = torch.from_numpy(W.special_values_f32().view(np.int32)).cuda()
    pick = torch.randint(0, words.shape[1], (4096,), generator=g, device="cuda")
    words[:, pick] = special[torch.arange(4096, device="cuda") % special.numel()]
    before = dense.clone()
    dst = torch.arange(cfg.n_req, dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix_windowed(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), [0, 3], layers=[0, 19],
                    label="windowed kda, raw bits", head_windows=True)
    keep = torch.from_numpy(mask_words(O).view(np.int32)).cuda()
    for j in range(cfg.n_req):
        a, b = dense[j].view(torch.int32), before[j].view(torch.int32)
        assert torch.equal(a & keep, b & keep), f"retained words of checkpoint {j}"


@pytest.mark.parametrize("w_max", [16, 64])
def test_windowed_equals_full_when_requests_fit_the_windows(w_max):
    # every head window is >= 4, so requests of at most 4 tokens replay the
    # same tokens on both entry points: bit-identical.  At W_max = 16 every
    # launch group's windows fit one chunk (the one-chunk kernel for every
    # width and gate layout), at 64 some do and some do not.
    cfg = W.Config("widths", _odd_refresh_layers(23), w_max=w_max, n_req=4, seed=23)
    P, O = _plans(cfg)
    assert min(O.head_window(li, int(h)) for li in range(len(cfg.layers))
               for h in O.refreshed_heads(li)) >= 4
    Wn = np.array([0, 1, 3, 4])
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    base = W.dense_states(cfg, 4, device="cuda", seed=11)
    a, b = base.clone(), base.clone()
    dst = torch.tensor([2, 0, 3, 1], dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, a, dst)
    R.ckpt_refresh_suffix_windowed(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, b, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    assert torch.equal(a, b)
    assert not torch.equal(a, base)


def _fused_vs_two_step(cfg, P, n_req, windows, seed, head_windows):
    Wn = np.asarray(windows)
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    n_ck = n_req + 1
    dense = W.dense_states(cfg, n_ck, device="cuda", seed=seed)
    info = P.info()
    pool = torch.zeros((n_ck, info["slot_bytes"]), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(seed)
    idx = torch.arange(n_ck, dtype=torch.int32, device="cuda")
    R.ckpt_pack(P, dense, idx, pool, idx)
    src_slot = torch.from_numpy(rng.permutation(n_ck)[:n_req].astype(np.int32)).cuda()
    dst = torch.from_numpy(rng.permutation(n_ck)[:n_req].astype(np.int32)).cuda()
    two = torch.full_like(dense, 0xA5)
    R.ckpt_unpack_zero_fill(P, pool, src_slot, two, dst)
    refresh = R.ckpt_refresh_suffix_windowed if head_windows else R.ckpt_refresh_suffix
    refresh(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, two, dst)
    one = torch.full_like(dense, 0x5A)
    R.ckpt_unpack_refresh(P, pool, src_slot, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, one, dst,
                          head_windows=head_windows)
    torch.cuda.synchronize()
    assert P.status() == 0
    d = dst.cpu().numpy()
    for r in range(n_req):
        assert torch.equal(one[int(d[r])], two[int(d[r])]), f"request {r}"
    return inp, pool, src_slot, dst, one


@pytest.mark.parametrize("head_windows", [False, True])
def test_fused_load_equals_unpack_then_refresh(head_windows):
    cases = [(W.tiny_kda(), [8, 3], 1),
             (W.Config("widths", _odd_refresh_layers(24), w_max=64, n_req=3, seed=24), [0, 21, 70], 2),
             (W.Config("widths", _odd_refresh_layers(26), w_max=16, n_req=3, seed=26), [2, 16, 33], 5),
             (W.kda_refresh(n_req=4), [256, 9, 16, 31], 3),
             (W.mixed(n_ckpt=8, n_req=3), [64, 200, 17], 4)]
    for cfg, windows, seed in cases:
        P, O = _plans(cfg)
        log(f"[fused] {cfg.name}: requests {windows}, head windows {head_windows}")
        _fused_vs_two_step(cfg, P, len(windows), windows, seed, head_windows)


@pytest.mark.parametrize("name,head_windows", [("tiny_kda", False), ("kda", False),
                                               ("kda", True), ("mixed", True)])
def test_fused_load_against_the_oracle(name, head_windows):
    # The fused dasc-wr load against the oracle itself (zero-fill unpack of
    # the slot, then the refresh over the request's tokens): retained units
    # and conv bytes bit-exact, the refreshed local units within the
    # tolerance; d = 128 KDA and GDN heads on the full-size layers, layers
    # sampled.
    if name == "tiny_kda":
        cfg, windows, layers = W.tiny_kda(), [8, 5], None
    elif name == "kda":
        cfg, windows, layers = W.kda_refresh(n_req=2), [256, 37], [0, 13]
    else:
        cfg, windows, layers = W.mixed(n_ckpt=4, n_req=2), [300, 64], [0, 1, 26]
    P, O = _plans(cfg)
    inp, pool, src_slot, dst, out = _fused_vs_two_step(cfg, P, 2, windows, 7, head_windows)
    tok = inp.tok_off.cpu().numpy()
    mask = mask_words(O)
    worst = 0.0
    for r in range(2):
        d, sl = int(dst[r]), int(src_slot[r])
        exp = np.full((1, O.dense_bytes), 0xEE, np.uint8)
        oracle.unpack_zero_fill(O, pool[sl:sl + 1].cpu().numpy(), [0], exp, [0])
        got = out[d].cpu().numpy()
        assert np.array_equal(got.view(np.uint32) & mask, exp[0].view(np.uint32) & mask)
        t0, t1 = int(tok[r]), int(tok[r + 1])
        ref = oracle.refresh_expected(O, _bits16(_host_rows(inp.k, (t0, t1))),
                                      _bits16(_host_rows(inp.v, (t0, t1))),
                                      _bits16(_host_rows(inp.a, (t0, t1))),
                                      _host_rows(inp.beta, (t0, t1)).numpy(),
                                      np.array([0, t1 - t0]), layers=layers,
                                      head_windows=head_windows)
        for (_, li, h), S64 in ref.items():
            local = local_mask_of_head(O, li, h)
            err = refresh_error(head_state(got, O, li, h), S64, local)
            worst = max(worst, err)
            assert err <= TOL, f"{name} req {r} layer {li} head {h}: {err:.3e}"
    log(f"[fused] {name} against the oracle: worst error {worst:.3e}")


def test_fused_load_bad_slot_is_flagged():
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    inp = W.refresh_inputs(cfg, np.array([8, 8]), device="cuda")
    pool = torch.zeros((2, P.info()["slot_bytes"]), dtype=torch.uint8, device="cuda")
    dense = torch.zeros((2, P.info()["dense_bytes"]), dtype=torch.uint8, device="cuda")
    bad = torch.tensor([0, 5], dtype=torch.int32, device="cuda")
    dst = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    R.ckpt_unpack_refresh(P, pool, bad, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() & R.STATUS_BAD_INDEX


# ---------------------------------------------------------------------------
# The recurrence's own form (token by token on the vector units), the
# reference point for the chunked kernel: the same tolerance against the
# fp64 oracle, and close to the chunked kernel's output.


def test_recurrent_every_width_against_the_oracle():
    cfg = W.Config("widths", _odd_refresh_layers(27), w_max=8, n_req=4, seed=27)
    P, O = _plans(cfg)
    Wn = np.array([0, 5, 16, 37])
    log(f"[recurrent] widths 16..128, GDN and KDA, requests {list(Wn)}")
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    dense = W.dense_states(cfg, 5, device="cuda", seed=13)
    before = dense.clone()
    dst = torch.tensor([4, 0, 3, 1], dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix_recurrent(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    assert torch.equal(dense[2], before[2])                 # not a destination
    _check_requests(P, O, inp, before, dense, dst.cpu().numpy(), range(4), label="recurrent")


def test_recurrent_kda_full_size_against_oracle_and_chunked():
    cfg = W.kda_refresh(n_req=16)
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    base = W.dense_states(cfg, cfg.n_req, device="cuda", seed=15)
    rec, chk = base.clone(), base.clone()
    dst = torch.from_numpy(np.random.default_rng(2).permutation(cfg.n_req).astype(np.int32)).cuda()
    R.ckpt_refresh_suffix_recurrent(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, rec, dst)
    R.ckpt_refresh_suffix(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, chk, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    _check_requests(P, O, inp, base, rec, dst.cpu().numpy(), [0, 11], layers=[0, 19],
                    label="recurrent kda")
    # both within 1e-4 of the oracle: within 2e-4 of each other, head by head
    worst = 0.0
    for li in (3, 12):
        L = O.layers[li]
        hb = L.d_v * L.d_k * 4
        for h in O.refreshed_heads(li)[:8]:
            local = local_mask_of_head(O, li, int(h))
            a0 = O.temporal_off[li] + int(h) * hb
            A = rec[:, a0:a0 + hb].cpu().numpy().view(np.float32).reshape(-1, L.d_v, L.d_k)
            Bc = chk[:, a0:a0 + hb].cpu().numpy().view(np.float32).reshape(-1, L.d_v, L.d_k)
            for d in range(cfg.n_req):
                a_, b_ = A[d].astype(np.float64), Bc[d].astype(np.float64)
                e = float(np.max(np.abs(a_[local] - b_[local])) / max(np.linalg.norm(b_), 1e-30))
                worst = max(worst, e)
    log(f"[recurrent] kda: recurrent vs chunked worst {worst:.3e}")
    assert worst <= 2 * TOL
