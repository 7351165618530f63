"""Oracle: bounded-suffix refresh, dasc-wr (test infrastructure only).

[dasc] §4.2 (load policies): the dasc-wr load rebuilds the omitted (local)
units of a compressed hit by running the recurrence over the last few
tokens, starting from an all-zero state of its own, and then overwrites
only those local units in the restored state; the pool slot is not
modified.

The recurrence is [dasc] §3.1 Eq. 1, with S in R^{d_v x d_k}:

    S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T

Expanding the product gives the rank-1 form used here:

    S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T)
        = S_{t-1} Diag(alpha_t) - beta_t (S_{t-1} Diag(alpha_t) k_t) k_t^T,

so S_t = A + beta_t (v_t - A k_t) k_t^T with A = S_{t-1} Diag(alpha_t).
For GDN the decay is one scalar per head and token, Diag(alpha_t) =
alpha_t I ([dasc] §3.1: GDN gates per head, KDA per channel).

The decays alpha_t enter in one of two ways:

* given directly, as Eq. 1 is written: fp32 alpha [T, sum_l (H d_k for
  KDA, H for GDN)], upcast exactly to float64;
* from the model's gate, [dasc] §3.3 Eq. 2 with the token's own logit a_t
  in place of the static a_s: alpha_t = exp(g_t), g_t = -exp(A_log)
  softplus(a_t + dt_bias), with a_t given as raw bf16 bits in a row of the
  same width.

Other inputs (token-major rows over the concatenated tokens of all
requests; the layer blocks follow one another in layer order, heads in
order inside): k [T, sum_l H d_k] and v [T, sum_l H d_v] as raw bf16 bits,
beta [T, sum_l H] float32, token offsets [n+1].  Everything is upcast
exactly to float64.
"""
from __future__ import annotations

import numpy as np

from .plan import GDN, OraclePlan, gate_log_decay


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (bf16 is the top half of an
    IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def delta_rule_step(S, alpha, beta, k, v):
    """One step of Eq. 1 in rank-1 form, float64.

    S [..., d_v, d_k]; alpha [..., d_k] (a GDN scalar is passed already
    broadcast over d_k); beta [...]; k [..., d_k]; v [..., d_v].
    """
    A = S * alpha[..., None, :]                      # S_{t-1} Diag(alpha_t)
    Ak = np.einsum("...ij,...j->...i", A, k)         # A k_t
    c = beta[..., None] * (v - Ak)                   # beta_t (v_t - A k_t)
    return A + c[..., :, None] * k[..., None, :]     # A + c k_t^T


def replay_rank1(alphas, betas, ks, vs, S0=None):
    """Replay Eq. 1 over W tokens from S0 (zero if None); leading axis of
    every input is the token."""
    W = len(betas)
    d_v, d_k = vs.shape[-1], ks.shape[-1]
    S = np.zeros(ks.shape[1:-1] + (d_v, d_k)) if S0 is None else np.array(S0, dtype=np.float64)
    for t in range(W):
        S = delta_rule_step(S, alphas[t], betas[t], ks[t], vs[t])
    return S


def replay_dense(alphas, betas, ks, vs, S0=None):
    """Eq. 1 exactly as printed, with dense matrices, for one head (tiny
    sizes only): S <- S @ Diag(alpha) @ (I - beta k k^T) + beta v k^T."""
    d_v, d_k = vs.shape[-1], ks.shape[-1]
    S = np.zeros((d_v, d_k)) if S0 is None else np.array(S0, dtype=np.float64)
    I = np.eye(d_k)
    for t in range(len(betas)):
        k = ks[t].reshape(d_k, 1)
        v = vs[t].reshape(d_v, 1)
        S = S @ np.diag(alphas[t]) @ (I - betas[t] * (k @ k.T)) + betas[t] * (v @ k.T)
    return S


def _row_offsets(plan: OraclePlan):
    """Where each layer's block starts inside a k / v / a / beta row."""
    ko, vo, go, bo = [], [], [], []
    k = v = g = b = 0
    for lay in plan.layers:
        ko.append(k); vo.append(v); go.append(g); bo.append(b)
        k += lay.n_heads * lay.d_k
        v += lay.n_heads * lay.d_v
        g += lay.n_heads * lay.d_k if lay.kind != GDN else lay.n_heads
        b += lay.n_heads
    return ko, vo, go, bo


def refresh_expected(plan: OraclePlan, k_bits, v_bits, a_bits, beta, tok_off,
                     requests=None, layers=None, heads=None, head_windows=False, alpha=None):
    """Scratch states of the bounded-suffix refresh, float64.

    For each request r (all, or the given subset), each layer (all, or the
    given subset) and each head the plan replays in that layer (optionally
    restricted to `heads`), start from S = 0 and apply Eq. 1 over the
    request's tokens tok_off[r] .. tok_off[r+1]-1.  With head_windows, head
    (l, h) replays only the last min(W_lh, n_r) of them, W_lh being the
    head's own Eq. 7 window ([dasc-sum] "Methodology" Eq. 7, taken per head
    rather than as one W_replay for the whole model).

    alpha: None to take each token's decays from its gate logits a_bits
    (Eq. 2), or fp32 decays [T, gate row] given directly (Eq. 1 as
    written; a_bits is then not read and may be None).

    Returns {(r, layer, head): S [d_v, d_k] float64}.  Only the local units
    of each S are written into the active state by the refresh.
    """
    ko, vo, go, bo = _row_offsets(plan)
    beta = np.asarray(beta, dtype=np.float32)
    if alpha is not None:
        alpha = np.asarray(alpha, dtype=np.float32)
    tok_off = np.asarray(tok_off, dtype=np.int64)
    n = len(tok_off) - 1
    out = {}
    for r in (range(n) if requests is None else requests):
        for li in (range(len(plan.layers)) if layers is None else layers):
            hs_all = plan.refreshed_heads(li)
            if heads is not None:
                hs_all = np.array([h for h in hs_all if h in set(heads)], dtype=np.int64)
            if len(hs_all) == 0:
                continue
            # heads that share a token range are replayed together
            t1 = int(tok_off[r + 1])
            starts = np.full(len(hs_all), int(tok_off[r]), dtype=np.int64)
            if head_windows:
                w = np.array([plan.head_window(li, int(h)) for h in hs_all], dtype=np.int64)
                starts = np.maximum(starts, t1 - w)
            for t0 in np.unique(starts):
                out.update(_replay_heads(plan, li, hs_all[starts == t0], int(t0), t1, r,
                                         k_bits, v_bits, a_bits, beta, ko, vo, go, bo, alpha))
    return out


def _replay_heads(plan, li, hs, t0, t1, r, k_bits, v_bits, a_bits, beta, ko, vo, go, bo,
                  alpha=None):
    """Eq. 1 from S = 0 over tokens t0 .. t1-1 for heads hs of layer li; the
    decays are read from alpha when given, else made from a_bits by Eq. 2."""
    out = {}
    lay = plan.layers[li]
    H, dk, dv = lay.n_heads, lay.d_k, lay.d_v
    ks = bf16_bits_to_f64(k_bits[t0:t1, ko[li]:ko[li] + H * dk]).reshape(-1, H, dk)[:, hs]
    vs = bf16_bits_to_f64(v_bits[t0:t1, vo[li]:vo[li] + H * dv]).reshape(-1, H, dv)[:, hs]
    bs = beta[t0:t1, bo[li]:bo[li] + H].astype(np.float64)[:, hs]
    if alpha is not None and lay.kind == GDN:
        al = alpha[t0:t1, go[li]:go[li] + H].astype(np.float64)[:, hs]   # [W, nh]
        al = np.repeat(al[:, :, None], dk, axis=2)                       # alpha_t I
    elif alpha is not None:
        al = alpha[t0:t1, go[li]:go[li] + H * dk].astype(np.float64).reshape(-1, H, dk)[:, hs]
    elif lay.kind == GDN:
        a = bf16_bits_to_f64(a_bits[t0:t1, go[li]:go[li] + H])[:, hs]
        g = gate_log_decay(lay.A_log[hs], lay.dt_bias[hs], a)      # [W, nh]
        al = np.repeat(np.exp(g)[:, :, None], dk, axis=2)          # alpha_t I
    else:
        a = bf16_bits_to_f64(a_bits[t0:t1, go[li]:go[li] + H * dk]).reshape(-1, H, dk)[:, hs]
        Al = lay.A_log.reshape(H, dk)[hs]
        Db = lay.dt_bias.reshape(H, dk)[hs]
        al = np.exp(gate_log_decay(Al, Db, a))                    # [W, nh, dk]
    S = replay_rank1(al, bs, ks, vs)
    for i, h in enumerate(hs):
        out[(r, li, int(h))] = S[i]
    return out
