"""GPU parity of the refresh that takes its decays directly (fp32 alpha, Eq. 1
as written), against the fp64 oracle fed the same fp32 decays, through the
C ABI; plus the one-hot-write-then-decay closed form on the GPU path.  The
error metric is the refresh's: max |S_gpu - S_fp64| over the written (local)
entries, over the Frobenius norm of the fp64 scratch state, <= 1e-4; the
bytes the refresh must not touch are compared bit for bit."""
import ctypes

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


def _bits16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _inputs(cfg, Wn, device):
    inp = W.refresh_inputs(cfg, Wn, device=device)
    alpha = W.refresh_decays(cfg, int(np.sum(Wn)), device=device)
    return inp, alpha


def _check(O, inp, alpha, before, after, dst, reqs, layers=None, label="", head_windows=False):
    tok = inp.tok_off.cpu().numpy()
    mask = mask_words(O)
    worst = 0.0
    for r in reqs:
        t0, t1 = int(tok[r]), int(tok[r + 1])
        k = _bits16(inp.k[t0:t1].cpu())
        v = _bits16(inp.v[t0:t1].cpu())
        al = alpha[t0:t1].cpu().numpy()
        b = inp.beta[t0:t1].cpu().numpy()
        ref = oracle.refresh_expected(O, k, v, None, b, np.array([0, t1 - t0]), layers=layers,
                                      head_windows=head_windows, alpha=al)
        d = int(dst[r])
        got = after[d].cpu().numpy()
        old = before[d].cpu().numpy()
        assert np.array_equal(got.view(np.uint32) & mask, old.view(np.uint32) & mask), f"req {r}"
        for (_, li, h), S64 in ref.items():
            local = local_mask_of_head(O, li, h)
            g = head_state(got, O, li, h)
            assert np.all(np.isfinite(g[local]))
            err = refresh_error(g, S64, local)
            worst = max(worst, err)
            assert err <= TOL, f"{label} req {r} layer {li} head {h}: {err:.3e}"
    log(f"[refresh alpha] {label}: worst error {worst:.3e} over requests {list(reqs)}")
    return worst


def test_alpha_tiny_kda_all_heads():
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp, alpha = _inputs(cfg, Wn, "cpu")
    inp = W.RefreshInputs(*(x.cuda() for x in (inp.k, inp.v, inp.a, inp.beta, inp.tok_off)))
    alpha = alpha.cuda()
    dense = W.dense_states(cfg, 3, device="cuda", seed=99)
    before = dense.clone()
    dst = torch.tensor([2, 0], dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix_alpha(P, inp.k, inp.v, alpha, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    assert torch.equal(dense[1], before[1])
    _check(O, inp, alpha, before, dense, dst.cpu().numpy(), [0, 1], label="tiny")


def test_alpha_kda_full_size_sampled():
    cfg = W.kda_refresh()
    log(f"[refresh alpha] kda: {cfg.n_req} requests x {cfg.window[0]} tokens")
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp, alpha = _inputs(cfg, Wn, "cuda")
    dense = W.dense_states(cfg, cfg.n_req, device="cuda", seed=5)
    before = dense.clone()
    dst = torch.from_numpy(np.random.default_rng(1).permutation(cfg.n_req).astype(np.int32)).cuda()
    R.ckpt_refresh_suffix_alpha(P, inp.k, inp.v, alpha, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    _check(O, inp, alpha, before, dense, dst.cpu().numpy(), [0, 37], layers=[0, 19], label="kda")
    _check(O, inp, alpha, before, dense, dst.cpu().numpy(), [63], layers=[9], label="kda")


def test_alpha_mixed_sampled():
    cfg = W.mixed(n_ckpt=64)
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    log(f"[refresh alpha] mixed: windows {Wn.min()}..{Wn.max()}, {int(Wn.sum())} tokens")
    inp, alpha = _inputs(cfg, Wn, "cuda")
    dense = W.dense_states(cfg, cfg.n_req, device="cuda", seed=6)
    before = dense.clone()
    dst = torch.arange(cfg.n_req, dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix_alpha(P, inp.k, inp.v, alpha, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    reqs = [int(np.argmax(Wn)), int(np.argmin(Wn))]
    _check(O, inp, alpha, before, dense, dst.cpu().numpy(), reqs, layers=[0, 1, 26],
           label="mixed")


def _odd_layers(seed):
    """Every refresh width (16, 32, 64, 128) as GDN and KDA layers, with KDA
    gate blocks on and off a 16-byte boundary (vector and element reads)."""
    rng = np.random.default_rng(seed)
    f = np.float32

    def lay(kind, H, d):
        n = H * d if kind == W.KDA else H
        A = rng.uniform(-1, 2, n) if kind == W.GDN else rng.normal(0, 1.5, n)
        return W.Layer(kind, H, d, d, A.astype(f), rng.normal(0, 1, n).astype(f), 0)

    return [lay(W.KDA, 2, 32), lay(W.GDN, 3, 32), lay(W.KDA, 2, 64), lay(W.GDN, 2, 64),
            lay(W.KDA, 1, 16), lay(W.GDN, 3, 16), lay(W.KDA, 2, 128), lay(W.GDN, 8, 16)]


@pytest.mark.parametrize("windowed", [False, True])
def test_alpha_every_width_and_unaligned_rows(windowed):
    cfg = W.Config("widths", _odd_layers(23), w_max=8, n_req=4, seed=23)
    P, O = _plans(cfg)
    kda_offsets = [P.layer(l)["gate_row_offset"] for l in range(len(cfg.layers))
                   if cfg.layers[l].kind == W.KDA]
    assert [o % 8 == 0 for o in kda_offsets] == [True, False, False, True], kda_offsets
    Wn = np.array([1, 17, 40, 100], dtype=np.int64)     # ragged: partial chunks
    inp, alpha = _inputs(cfg, Wn, "cuda")
    dense = W.dense_states(cfg, 5, device="cuda", seed=7)
    before = dense.clone()
    dst = torch.tensor([4, 1, 0, 3], dtype=torch.int32, device="cuda")
    fn = R.ckpt_refresh_suffix_alpha_windowed if windowed else R.ckpt_refresh_suffix_alpha
    fn(P, inp.k, inp.v, alpha, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    assert torch.equal(dense[2], before[2])
    _check(O, inp, alpha, before, dense, dst.cpu().numpy(), range(4),
           label="widths windowed" if windowed else "widths", head_windows=windowed)


def test_alpha_windowed_kda_sampled():
    cfg = W.kda_refresh(n_req=16)
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp, alpha = _inputs(cfg, Wn, "cuda")
    dense = W.dense_states(cfg, cfg.n_req, device="cuda", seed=8)
    before = dense.clone()
    dst = torch.arange(cfg.n_req, dtype=torch.int32, device="cuda")
    R.ckpt_refresh_suffix_alpha_windowed(P, inp.k, inp.v, alpha, inp.beta, inp.tok_off, dense,
                                         dst)
    torch.cuda.synchronize()
    assert P.status() == 0
    _check(O, inp, alpha, before, dense, dst.cpu().numpy(), [3, 15], layers=[0, 11],
           label="kda windowed", head_windows=True)


@pytest.mark.parametrize("kind,d", [(W.KDA, 128), (W.GDN, 128), (W.KDA, 32), (W.GDN, 16)])
def test_one_hot_write_then_constant_decay_closed_form(kind, d):
    # From the zero scratch state: token j < d writes v_j into column j
    # (k = e_j, beta = 1; the write removes what the column held); every
    # later token multiplies column j by its decay.  With alpha = 0.97
    # everywhere and beta = 0 after the write phase, column j ends as
    # v_j 0.97^(W - 1 - j) after W = 256 tokens, in closed form and
    # independently of the oracle.  Every unit is local (short horizons).
    H, T, a = 4, 256, 0.97
    n = H * d if kind == W.KDA else H
    lay = W.Layer(kind, H, d, d, np.full(n, 2.0, np.float32), np.zeros(n, np.float32), 0)
    cfg = W.Config("onehot", [lay], w_max=64)
    P, O = _plans(cfg)
    assert len(O.refreshed_heads(0)) == H and not O.layers[0].retained.any()
    k = np.zeros((T, H, d), np.float32)
    for j in range(d):
        k[j, :, j] = 1.0
    rng = np.random.default_rng(40 + d)
    v = rng.normal(0, 1, (T, H * d)).astype(np.float32)
    kt = torch.from_numpy(k.reshape(T, H * d)).to(torch.bfloat16).cuda()
    vt = torch.from_numpy(v).to(torch.bfloat16).cuda()
    alpha = torch.full((T, n), a, dtype=torch.float32, device="cuda")
    beta = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    beta[:d] = 1.0
    dense = torch.full((2, O.dense_bytes), 0x7F, dtype=torch.uint8, device="cuda")
    R.ckpt_refresh_suffix_alpha(P, kt, vt, alpha, beta, torch.tensor([0, T], device="cuda"),
                                dense, torch.tensor([1], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert P.status() == 0
    assert torch.all(dense[0] == 0x7F)
    row = dense[1].cpu().numpy()
    vb = vt.float().cpu().numpy().astype(np.float64)
    a32 = float(np.float32(a))
    worst = 0.0
    for h in range(H):
        S = head_state(row, O, 0, h).astype(np.float64)
        expect = np.zeros((d, d))
        for j in range(d):
            expect[:, j] = vb[j, h * d:(h + 1) * d] * a32 ** (T - 1 - j)
        err = np.max(np.abs(S - expect)) / np.linalg.norm(expect)
        worst = max(worst, err)
        assert err <= TOL, f"head {h}: {err:.3e}"
    log(f"[refresh alpha] one-hot write then decay, kind {kind} d {d}: worst error {worst:.3e}")


def test_alpha_rejects_misaligned_and_null_decays():
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp, alpha = _inputs(cfg, Wn, "cuda")
    dense = W.dense_states(cfg, 2, device="cuda", seed=9)
    before = dense.clone()
    dst = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    flat = torch.zeros(alpha.numel() + 1, dtype=torch.float32, device="cuda")
    off = flat[1:].view(alpha.shape)                    # contiguous, 4-byte aligned only
    with pytest.raises(R.DascError, match="16-byte aligned"):
        R.ckpt_refresh_suffix_alpha(P, inp.k, inp.v, off, inp.beta, inp.tok_off, dense, dst)
    with pytest.raises(TypeError):                      # bf16 logits are not decays
        R.ckpt_refresh_suffix_alpha(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, dense, dst)
    torch.cuda.synchronize()
    assert torch.equal(dense, before)


@pytest.mark.parametrize("kind,d", [(W.KDA, 128), (W.GDN, 128), (W.KDA, 32), (W.GDN, 16)])
def test_one_repeated_key_keeps_only_the_last_value(kind, d):
    # Every token writes with the same unit key k (bf16-exact), beta = 1 and
    # decay 1: each write replaces the whole state, S_t = v_t k^T ([dasc]
    # §3.1 Eq. 1 with alpha = 1: S (I - k k^T) + v k^T and S = v' k^T gives
    # v k^T).  Inside a chunk every entry of L is 1, the worst case of the
    # inverse (its 8 x 8 blocks and their coupling block included); 40
    # tokens span two full chunks and a partial one.  Independent of the
    # oracle.
    H, T = 4, 40
    n = H * d if kind == W.KDA else H
    lay = W.Layer(kind, H, d, d, np.full(n, 2.0, np.float32), np.zeros(n, np.float32), 0)
    cfg = W.Config("repeat", [lay], w_max=64, seed=43)
    P, O = _plans(cfg)
    assert len(O.refreshed_heads(0)) == H and O.layers[0].r == 0
    rng = np.random.default_rng(11)
    key = np.zeros((H, d), np.float32)
    for h in range(H):
        idx = rng.choice(d, 16, replace=False)
        key[h, idx] = rng.choice([-0.25, 0.25], 16)
    kt = torch.from_numpy(np.broadcast_to(key.reshape(1, H * d), (T, H * d)).copy())
    kt = kt.to(torch.bfloat16).cuda()
    vt = torch.randn(T, H * d).to(torch.bfloat16).cuda()
    alpha = torch.ones(T, n, dtype=torch.float32, device="cuda")
    bt = torch.ones(T, H, dtype=torch.float32, device="cuda")
    dense = torch.zeros((1, O.dense_bytes), dtype=torch.uint8, device="cuda")
    R.ckpt_refresh_suffix_alpha(P, kt, vt, alpha, bt, torch.tensor([0, T], device="cuda"),
                                dense, torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert P.status() == 0
    row = dense[0].cpu().numpy()
    worst = 0.0
    for h in range(H):
        S = head_state(row, O, 0, h).astype(np.float64)
        vlast = vt[-1, h * d:(h + 1) * d].float().cpu().numpy().astype(np.float64)
        ref = np.outer(vlast, key[h].astype(np.float64))
        err = np.max(np.abs(S - ref)) / np.linalg.norm(ref)
        worst = max(worst, err)
        assert err <= TOL, f"head {h}: {err:.3e}"
    log(f"[refresh alpha] repeated key, kind {kind} d {d}: worst error {worst:.3e}")


def test_refresh_rejects_token_counts_from_2_31():
    # The kernels index tokens in 32 bits: the host refuses n_tokens >= 2^31
    # (DASC_EINVAL) before anything is launched.
    cfg = W.tiny_kda()
    P, O = _plans(cfg)
    Wn = W.windows(cfg)
    inp, alpha = _inputs(cfg, Wn, "cuda")
    dense = W.dense_states(cfg, 2, device="cuda", seed=9)
    before = dense.clone()
    dst = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    args = (ptr(inp.k), ptr(inp.v), ptr(alpha), ptr(inp.beta), ptr(inp.tok_off))
    tail = (ptr(dense), dense.stride(0), dense.shape[0], ptr(dst), 2, None)
    for n_tokens in (2 ** 31, 2 ** 40):
        assert R.lib.dasc_ckpt_refresh_suffix_alpha(P._h, *args, n_tokens, *tail) == -1
        assert R.lib.dasc_ckpt_refresh_suffix_alpha_windowed(P._h, *args, n_tokens, *tail) == -1
    assert R.lib.dasc_ckpt_refresh_suffix_alpha(P._h, *args, int(inp.k.shape[0]), *tail) == 0
    torch.cuda.synchronize()
    assert P.status() == 0
    assert not torch.equal(dense, before)


@pytest.mark.parametrize("kind", [W.KDA, W.GDN])
def test_alpha_recall_invariant(kind):
    # beta = 1 and keys of exactly unit norm in bf16 (+-1/4 on 16 of 128
    # coordinates): whatever the decays, the final state recalls the last
    # value, S_W k_W = v_W ([dasc] §3.1 Eq. 1), independently of the oracle.
    d, H, T = 128, 4, 40
    n = H * d if kind == W.KDA else H
    lay = W.Layer(kind, H, d, d, np.full(n, 2.0, np.float32), np.zeros(n, np.float32), 0)
    cfg = W.Config("recall", [lay], w_max=64, seed=41)
    P, O = _plans(cfg)
    assert len(O.refreshed_heads(0)) == H
    rng = np.random.default_rng(9)
    k = np.zeros((T, H, d), np.float32)
    for t in range(T):
        for h in range(H):
            idx = rng.choice(d, 16, replace=False)
            k[t, h, idx] = rng.choice([-0.25, 0.25], 16)
    kt = torch.from_numpy(k.reshape(T, H * d)).to(torch.bfloat16).cuda()
    vt = torch.randn(T, H * d).to(torch.bfloat16).cuda()
    alpha = W.refresh_decays(cfg, T, device="cuda")
    bt = torch.ones(T, H, dtype=torch.float32, device="cuda")
    dense = torch.zeros((1, O.dense_bytes), dtype=torch.uint8, device="cuda")
    R.ckpt_refresh_suffix_alpha(P, kt, vt, alpha, bt, torch.tensor([0, T], device="cuda"),
                                dense, torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert P.status() == 0
    row = dense[0].cpu().numpy()
    for h in range(H):
        S = head_state(row, O, 0, h).astype(np.float64)
        vlast = vt[-1, h * d:(h + 1) * d].float().cpu().numpy()
        recall = S @ k[-1, h].astype(np.float64)
        assert np.max(np.abs(recall - vlast)) <= 1e-5 * max(1.0, np.linalg.norm(vlast))
