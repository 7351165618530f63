"""Seeded synthetic inputs for the checkpoint hot path.

This module only draws random numbers and lays them out.  It holds none of
the arithmetic of the method (no decay gate, no horizon, no mask, no pack,
no recurrence): both the CPU oracle and the HIP library consume what it
produces, and neither is used here.

Shapes follow the recurrent layers described on the dasc pages:
Qwen3-Next has 36 Gated DeltaNet (GDN) layers and Kimi-Linear 20 Kimi Delta
Attention (KDA) layers ("5.1 Setup, Models and hardware"), key width 128
(Appendix A.1, Figure 5), 32 heads per layer, fp32 temporal state and bf16
convolution state ("4.1 Decay-aware selection and storage").

Layouts the generators produce (the library documents the same layouts):

* dense checkpoint: per layer l the temporal state [H, d_v, d_k] fp32
  (k fastest), layers back to back, then every layer's conv bytes back to
  back.  A batch of checkpoints is a uint8 tensor [n, dense_bytes].
* refresh inputs, token-major rows over the concatenated tokens of all
  requests: k [T, sum_l H*d_k] bf16, v [T, sum_l H*d_v] bf16,
  gate logits a [T, sum_l (H*d_k if KDA else H)] bf16,
  beta [T, sum_l H] fp32, token offsets [n+1] int64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

GDN = 0
KDA = 1

# Seeds per named configuration (the pages' Random-mask seeds, reused here
# only as seeds).
SEEDS = {"tiny_kda": 1234, "gdn": 2027, "kda": 3407, "kda_refresh": 4519, "mixed": 5683}


@dataclass
class Layer:
    kind: int            # GDN (head-wise units) or KDA (key-channel units)
    n_heads: int
    d_k: int
    d_v: int
    A_log: np.ndarray    # float32, [n_heads] (GDN) or [n_heads*d_k] (KDA)
    dt_bias: np.ndarray  # float32, same shape as A_log
    conv_bytes: int = 0  # bf16 conv-state bytes this layer adds to a checkpoint

    @property
    def gate_width(self) -> int:
        return self.n_heads * self.d_k if self.kind == KDA else self.n_heads


@dataclass
class Config:
    name: str
    layers: list
    w_max: int
    a_s: float = -0.3
    eps: float = 1e-3
    n_ckpt: int = 0          # checkpoints packed / unpacked per step
    n_req: int = 0           # refresh requests
    window: tuple = (0, 0)   # refresh window per request: fixed or U{lo..hi}
    state_std: float = 1.0
    seed: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def temporal_bytes(self) -> int:
        return sum(l.n_heads * l.d_v * l.d_k * 4 for l in self.layers)

    @property
    def conv_bytes(self) -> int:
        return sum(l.conv_bytes for l in self.layers)

    @property
    def dense_bytes(self) -> int:
        return self.temporal_bytes + self.conv_bytes


def _rng(seed: int, stream: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=seed + (stream << 32)))


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


# Per-layer conv state: 4 positions x (3 * heads * 128) bf16 channels.
def _conv_bytes(n_heads: int, d: int, positions: int = 4) -> int:
    return positions * 3 * n_heads * d * 2


def tiny_kda() -> Config:
    """1 KDA layer, 4 heads, d_k=d_v=16, A_log and dt_bias ~ N(0,1)."""
    seed = SEEDS["tiny_kda"]
    r = _rng(seed)
    H, d = 4, 16
    layer = Layer(KDA, H, d, d, _f32(r.standard_normal(H * d)),
                  _f32(r.standard_normal(H * d)), 0)
    return Config("tiny_kda", [layer], w_max=16, n_ckpt=2, n_req=2,
                  window=(8, 8), state_std=1.0, seed=seed)


def gdn(n_ckpt: int = 64) -> Config:
    """36 GDN layers x 32 heads, d=128, A_log ~ U(-1,2), dt_bias ~ N(0,1).

    W_max = 10 is the integer whose retained-head fraction is nearest 45%
    for these draws (a test re-derives it from the oracle plan).
    """
    seed = SEEDS["gdn"]
    r = _rng(seed)
    layers = [Layer(GDN, 32, 128, 128, _f32(r.uniform(-1.0, 2.0, 32)),
                    _f32(r.standard_normal(32)), 0) for _ in range(36)]
    return Config("gdn", layers, w_max=GDN_W_MAX, n_ckpt=n_ckpt,
                  state_std=0.05, seed=seed)


def kda(n_ckpt: int = 64, n_req: int = 64, window: int = 256) -> Config:
    """20 KDA layers x 32 heads, d=128, per-channel A_log ~ N(0, 1.5^2).

    dt_bias is the constant 0.416, which puts the median one-step decay at
    the static gate near 0.47 (the Kimi-Linear median the pages report).
    W_max = 14 is the integer whose retained-channel fraction is nearest
    38% (re-derived by a test); the pages' W_max = 16 would keep 35.4% here.
    Conv state 4 x (3*32*128) bf16 per layer.
    """
    seed = SEEDS["kda"]
    r = _rng(seed)
    layers = [Layer(KDA, 32, 128, 128, _f32(1.5 * r.standard_normal(32 * 128)),
                    _f32(np.full(32 * 128, 0.416)), _conv_bytes(32, 128))
              for _ in range(20)]
    return Config("kda", layers, w_max=KDA_W_MAX, n_ckpt=n_ckpt, n_req=n_req,
                  window=(window, window), state_std=1.0, seed=seed)


def kda_refresh(n_req: int = 64, window: int = 256) -> Config:
    """The KDA layers above, refreshing 64 requests of 256 tokens."""
    c = kda(n_ckpt=n_req, n_req=n_req, window=window)
    c.name = "kda_refresh"
    c.seed = SEEDS["kda_refresh"]
    return c


def mixed(n_ckpt: int = 512, n_req: int = 64) -> Config:
    """27 layers alternating GDN (even) and KDA (odd), 32 heads, d=128.

    Each layer gets a target retained fraction f_l ~ U(0.2, 0.8).  Exactly
    round(f_l * n_l) randomly chosen units draw a slow-decay A_log from
    U(-6, -2.5); the rest draw a fast-decay A_log from U(-1, 3); dt_bias = 0.
    At W_max = 64 the two populations fall on opposite sides of the
    threshold with a wide margin, so the plan retains exactly the slow ones.
    Conv state as in the KDA configuration, on every layer.
    """
    seed = SEEDS["mixed"]
    r = _rng(seed)
    layers, fracs = [], []
    for l in range(27):
        kind = GDN if l % 2 == 0 else KDA
        n = 32 if kind == GDN else 32 * 128
        f = float(r.uniform(0.2, 0.8))
        n_slow = int(round(f * n))
        slow = np.zeros(n, dtype=bool)
        slow[r.permutation(n)[:n_slow]] = True
        a_log = np.where(slow, r.uniform(-6.0, -2.5, n), r.uniform(-1.0, 3.0, n))
        layers.append(Layer(kind, 32, 128, 128, _f32(a_log), _f32(np.zeros(n)),
                            _conv_bytes(32, 128)))
        fracs.append(n_slow / n)
    return Config("mixed", layers, w_max=64, n_ckpt=n_ckpt, n_req=n_req,
                  window=(64, 1024), state_std=1.0, seed=seed,
                  extra={"slow_fraction": fracs})


# Integer thresholds picked for the draws above (verified by tests).
GDN_W_MAX = 10
KDA_W_MAX = 14

CONFIGS = {"tiny_kda": tiny_kda, "gdn": gdn, "kda": kda,
           "kda_refresh": kda_refresh, "mixed": mixed}


# ----------------------------------------------------------------------------
# Dense checkpoints and pool slot orders
# ----------------------------------------------------------------------------

def dense_states(cfg: Config, n: int, device="cpu", seed: int | None = None,
                 std: float | None = None) -> torch.Tensor:
    """n dense checkpoints as uint8 [n, dense_bytes].

    The temporal part is N(0, std^2) fp32, the conv part N(0,1) rounded to
    bf16.  Drawn with torch's generator on `device`.
    """
    seed = cfg.seed if seed is None else seed
    std = cfg.state_std if std is None else std
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((n, cfg.dense_bytes), dtype=torch.uint8, device=device)
    nt = cfg.temporal_bytes // 4
    for i in range(n):
        t = out[i, :cfg.temporal_bytes].view(torch.float32)
        torch.randn(nt, generator=g, device=device, out=t)
        t.mul_(std)
        if cfg.conv_bytes:
            c = torch.randn(cfg.conv_bytes // 2, generator=g, device=device)
            out[i, cfg.temporal_bytes:].view(torch.bfloat16).copy_(c)
    return out


def special_values_f32() -> np.ndarray:
    """fp32 bit patterns a raw copy must preserve: -0.0, NaNs with payloads,
    infinities, denormals, the smallest and largest normals."""
    return np.array([0x80000000, 0x7FC00001, 0xFFC12345, 0x7F800001,
                     0x7F800000, 0xFF800000, 0x00000001, 0x807FFFFF,
                     0x00800000, 0x7F7FFFFF, 0x3F800000, 0xBF800000],
                    dtype=np.uint32)


def slot_permutation(n: int, seed: int) -> np.ndarray:
    """A random order of n pool slots (the mixed configuration's ragged
    order)."""
    return _rng(seed, 7).permutation(n).astype(np.int32)


# ----------------------------------------------------------------------------
# Refresh inputs
# ----------------------------------------------------------------------------

def windows(cfg: Config, seed: int | None = None) -> np.ndarray:
    """Per-request suffix lengths: fixed, or uniform over {lo..hi}."""
    lo, hi = cfg.window
    if lo == hi:
        return np.full(cfg.n_req, lo, dtype=np.int64)
    r = _rng(cfg.seed if seed is None else seed, 3)
    return r.integers(lo, hi + 1, size=cfg.n_req).astype(np.int64)


@dataclass
class RefreshInputs:
    k: torch.Tensor        # bf16 [T, sum H*d_k]
    v: torch.Tensor        # bf16 [T, sum H*d_v]
    a: torch.Tensor        # bf16 [T, sum gate_width]
    beta: torch.Tensor     # fp32 [T, sum H]
    tok_off: torch.Tensor  # int64 [n+1]


def refresh_inputs(cfg: Config, W: np.ndarray, device="cpu",
                   seed: int | None = None) -> RefreshInputs:
    """k: each (token, layer, head) key drawn N(0,1) and scaled to unit L2
    norm, then rounded to bf16; v ~ N(0,1) and gate logits a ~ N(0,1),
    rounded to bf16; beta = sigmoid(N(0,1)) in fp32."""
    seed = cfg.seed if seed is None else seed
    g = torch.Generator(device=device)
    g.manual_seed(seed + 17)
    T = int(np.sum(W))
    kw = sum(l.n_heads * l.d_k for l in cfg.layers)
    vw = sum(l.n_heads * l.d_v for l in cfg.layers)
    gw = sum(l.gate_width for l in cfg.layers)
    bw = sum(l.n_heads for l in cfg.layers)
    k = torch.empty((T, kw), dtype=torch.bfloat16, device=device)
    off = 0
    for l in cfg.layers:
        w = l.n_heads * l.d_k
        x = torch.randn((T, l.n_heads, l.d_k), generator=g, device=device)
        x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        k[:, off:off + w] = x.reshape(T, w).to(torch.bfloat16)
        off += w
    v = torch.randn((T, vw), generator=g, device=device).to(torch.bfloat16)
    a = torch.randn((T, gw), generator=g, device=device).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((T, bw), generator=g, device=device))
    tok = torch.zeros(len(W) + 1, dtype=torch.int64)
    tok[1:] = torch.from_numpy(np.cumsum(W).astype(np.int64))
    return RefreshInputs(k, v, a, beta.contiguous(), tok.to(device))


def refresh_decays(cfg: Config, T: int, device="cpu", seed: int | None = None) -> torch.Tensor:
    """fp32 decays [T, sum gate_width] for the refresh that takes the decays
    directly: each unit (a KDA channel, or a GDN head) gets a floor
    f_u = x^3 with x ~ U(0, 1), drawn once, and each token the decay
    f_u + (1 - f_u) w with w ~ U(0, 1).  The median decay is near 0.67 (the
    pages' median one-step KDA decay is 0.47); the few units with a floor
    near 1 decay slowly over every token (long memories, which stress the
    accumulation over long windows), the many with a low floor see decays
    over most of (0, 1).  A plain random draw: these decays do not come
    from the model's gate."""
    seed = cfg.seed if seed is None else seed
    g = torch.Generator(device=device)
    g.manual_seed(seed + 29)
    gw = sum(l.gate_width for l in cfg.layers)
    floor = torch.rand((1, gw), generator=g, device=device) ** 3
    out = torch.empty((T, gw), dtype=torch.float32, device=device)
    step = 4096
    for t0 in range(0, T, step):
        w = torch.rand((min(step, T - t0), gw), generator=g, device=device)
        out[t0:t0 + w.shape[0]] = floor + (1.0 - floor) * w
    return out
