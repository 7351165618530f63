"""Oracle: the static selection plan (test infrastructure only).

Follows [dasc] §3.3 Eq. 2 and Eq. 3, §4.1, Appendix B "Ragged (Scheme 2)"
and "Padded (Scheme 1)", Appendix C.1 Eq. 8, and [dasc-sum] "Methodology"
Eq. 6 and Eq. 7.  All floating point is float64 on float32 inputs upcast.

Readings taken where the pages leave a step open:
* the static gate logit a_s is a parameter (the pages fix -0.3 for the
  Qwen3-Next / Kimi-Linear plans) and Eq. 2 is applied per unit: per head for
  GDN, per key channel (h, k) for KDA;
* a unit is retained iff H_s > W_max, strictly; a gate that underflows to
  g = -0 gives H_s = +inf (retained);
* next_pow2(x) is the smallest power of two >= x for x > 1, and 1 for x <= 1;
  clamp(x, 4, W_max) = min(max(x, 4), W_max), so W_max wins when below 4;
* W_replay = 0 when a plan has no local unit;
* offsets are 0-based exclusive prefix sums, o_0 = 0, o_{l+1} = o_l + r_l;
* units are ordered by ascending head index (GDN) or h*d_k + k (KDA),
  layers in increasing order; the checkpoint's conv bytes follow the whole
  temporal payload, in layer order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GDN = 0
KDA = 1


def softplus(x: np.ndarray) -> np.ndarray:
    """softplus(x) = ln(1 + e^x), evaluated without overflow (float64)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def gate_log_decay(A_log, dt_bias, a) -> np.ndarray:
    """[dasc] §3.3 Eq. 2: g = -exp(A_log) * softplus(a + dt_bias)."""
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    return -np.exp(A_log) * softplus(a + dt_bias)


def horizon(g, eps: float) -> np.ndarray:
    """[dasc] §3.3 Eq. 3: H_s = ln(eps) / g, the number of tokens after which
    the static decay factor exp(g * tokens) has fallen to eps."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.float64(math.log(eps)) / g


def next_pow2(x: float) -> int:
    """Smallest power of two >= x (1 for x <= 1 or NaN), by doubling."""
    p = 1
    if not (x > 1.0):
        return 1
    while p < x:
        p *= 2
    return p


def replay_window(H_s: float, w_max: int) -> int:
    """[dasc-sum] "Methodology" Eq. 7, per local unit:
    W_u = clamp(next_pow2(H_s(u)), 4, W_max)."""
    return min(max(next_pow2(H_s), 4), w_max)


def slots_eq8(budget_bytes: int, slot_bytes: int) -> int:
    """[dasc] Appendix C.1 Eq. 8 on one rank: floor(B / b_full) - 1, the
    subtracted slot being the allocator's reserved slot 0."""
    return budget_bytes // slot_bytes - 1


@dataclass
class OracleLayer:
    kind: int
    n_heads: int
    d_k: int
    d_v: int
    conv_bytes: int
    g: np.ndarray          # per unit, float64
    H_s: np.ndarray        # per unit, float64
    retained: np.ndarray   # per unit, bool
    retained_idx: np.ndarray
    local_idx: np.ndarray
    W_u: np.ndarray        # per local unit (aligned with local_idx), int64
    A_log: np.ndarray      # float32 per unit (as given)
    dt_bias: np.ndarray

    @property
    def n(self) -> int:           # n_l, total units
        return len(self.retained)

    @property
    def r(self) -> int:           # r_l, retained units
        return int(len(self.retained_idx))

    @property
    def unit_bytes(self) -> int:  # a GDN head state, or one KDA column
        return (self.d_v * self.d_k * 4) if self.kind == GDN else self.d_v * 4

    @property
    def state_bytes(self) -> int:
        return self.n_heads * self.d_v * self.d_k * 4


@dataclass
class OraclePlan:
    layers: list
    a_s: float
    eps: float
    w_max: int
    unit_off: list = field(default_factory=list)     # o_l, in units
    temporal_off: list = field(default_factory=list)  # bytes in a dense ckpt
    conv_off: list = field(default_factory=list)      # bytes in a dense ckpt
    pool_off: list = field(default_factory=list)      # bytes in a pool slot
    pool_conv_off: list = field(default_factory=list)  # bytes in a pool slot
    B_temp_dense: int = 0
    B_temp_rag: int = 0
    B_conv: int = 0
    W_replay: int = 0
    W_layer: list = field(default_factory=list)       # max W_u per layer

    @property
    def dense_bytes(self) -> int:
        return self.B_temp_dense + self.B_conv

    @property
    def slot_bytes(self) -> int:
        return self.B_temp_rag + self.B_conv

    # [dasc-sum] Eq. 6, temporal ratio (unit counts), and the complete
    # checkpoint ratio from byte counts.
    @property
    def C_temp(self) -> float:
        rs = sum(l.r for l in self.layers)
        return math.inf if rs == 0 else sum(l.n for l in self.layers) / rs

    @property
    def C_ckpt(self) -> float:
        den = self.B_temp_rag + self.B_conv
        return math.inf if den == 0 else (self.B_temp_dense + self.B_conv) / den

    # [dasc] §4.1 / Appendix B "Padded (Scheme 1)".
    @property
    def R_max(self) -> int:
        return max(l.r for l in self.layers)

    @property
    def r_bar(self) -> float:
        return sum(l.r for l in self.layers) / len(self.layers)

    @property
    def C_temp_pad(self) -> float:
        L = len(self.layers)
        return math.inf if self.R_max == 0 else sum(l.n for l in self.layers) / (L * self.R_max)

    @property
    def C_temp_rag(self) -> float:
        """Appendix B "Ragged (Scheme 2)": (sum n_l) / (L * r_bar)."""
        L = len(self.layers)
        return math.inf if self.r_bar == 0 else sum(l.n for l in self.layers) / (L * self.r_bar)

    def refreshed_heads(self, li: int) -> np.ndarray:
        """Heads a bounded-suffix refresh must replay in layer li: GDN local
        heads; KDA heads with at least one local channel (the whole head is
        replayed because (I - beta k k^T) couples its columns)."""
        lay = self.layers[li]
        if lay.kind == GDN:
            return np.flatnonzero(~lay.retained)
        per_head = lay.retained.reshape(lay.n_heads, lay.d_k)
        return np.flatnonzero(~per_head.all(axis=1))

    def head_window(self, li: int, h: int) -> int:
        """Eq. 7 window of one replayed head: the largest W_u over the
        head's local units (a GDN local head is one unit; a KDA head's local
        channels share one replay, because (I - beta k k^T) couples the
        columns).  0 for a head with no local unit."""
        lay = self.layers[li]
        if lay.kind == GDN:
            sel = lay.local_idx == h
        else:
            sel = (lay.local_idx // lay.d_k) == h
        return int(lay.W_u[sel].max()) if sel.any() else 0


def build_plan(layers, a_s: float = -0.3, eps: float = 1e-3,
               w_max: int = 16) -> OraclePlan:
    """Static selection plan ([dasc] §4.1): per unit u of every layer,
    g_u from Eq. 2 at the fixed logit a = a_s, H_s(u) from Eq. 3, retain
    iff H_s(u) > W_max; ragged offsets (Appendix B, Scheme 2); per local
    unit the Eq. 7 window; byte totals.

    `layers` is a sequence of objects with kind, n_heads, d_k, d_v, A_log,
    dt_bias and conv_bytes (A_log / dt_bias: float32, one per unit).
    """
    out_layers = []
    for lay in layers:
        n_units = lay.n_heads if lay.kind == GDN else lay.n_heads * lay.d_k
        A = np.asarray(lay.A_log, dtype=np.float32).reshape(-1)
        D = np.asarray(lay.dt_bias, dtype=np.float32).reshape(-1)
        assert A.shape == (n_units,) and D.shape == (n_units,)
        g = gate_log_decay(A, D, a_s)
        H = horizon(g, eps)
        retained = H > w_max
        ret_idx = np.flatnonzero(retained).astype(np.int64)
        loc_idx = np.flatnonzero(~retained).astype(np.int64)
        W_u = np.array([replay_window(float(H[u]), w_max) for u in loc_idx],
                       dtype=np.int64)
        out_layers.append(OracleLayer(lay.kind, lay.n_heads, lay.d_k, lay.d_v,
                                      int(lay.conv_bytes), g, H, retained,
                                      ret_idx, loc_idx, W_u, A, D))
    plan = OraclePlan(out_layers, a_s, eps, w_max)

    o = 0
    t_off = 0
    p_off = 0
    for lay in out_layers:
        plan.unit_off.append(o)
        plan.temporal_off.append(t_off)
        plan.pool_off.append(p_off)
        o += lay.r
        t_off += lay.state_bytes
        p_off += lay.r * lay.unit_bytes
    plan.unit_off.append(o)
    plan.B_temp_dense = t_off
    plan.B_temp_rag = p_off
    c_dense = t_off
    c_pool = p_off
    for lay in out_layers:
        plan.conv_off.append(c_dense)
        plan.pool_conv_off.append(c_pool)
        c_dense += lay.conv_bytes
        c_pool += lay.conv_bytes
    plan.B_conv = sum(l.conv_bytes for l in out_layers)
    plan.W_layer = [int(l.W_u.max()) if len(l.W_u) else 0 for l in out_layers]
    plan.W_replay = max(plan.W_layer) if plan.W_layer else 0
    return plan
