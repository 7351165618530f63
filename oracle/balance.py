"""Oracle: tensor-parallel storage balancing (test infrastructure only).

[dasc] §4.3 "TP-balanced placement" and Appendix B.1 "Deterministic TP
balancing", part (b) "State checkpoint storage balancing".  Under tensor
parallelism of degree P every rank owns whole heads and packs the retained
units of its own heads (its compute-local units, n_r of them, in its ragged
order: layer by layer, unit by unit).  Storage balancing redistributes the
packed units so that every rank stores about the same number:

* N = sum_r n_r and (q, m) = divmod(N, P);
* ranks sorted by (-n_r, r): the first m get the target t_r = q + 1, the
  rest t_r = q;
* rank r keeps its first min(n_r, t_r) units;
* excess units, listed by source rank and then local unit index, are paired
  in order with deficit positions, listed by destination rank and then
  position;
* every rank allocates ceil(N / P) units per slot;
* M_remote = sum_r max(0, n_r - t_r) units cross ranks, each exactly once.

Store: compute-local state -> pack and partition -> variable-split
all-to-all -> scatter into the storage slots.  Load runs the inverse.

Readings (the pages leave them open):
* A rank's compute-local heads are the contiguous block
  [r H / P, (r + 1) H / P) of every layer (no compute-head permutation), and
  its conv bytes are the layer's conv bytes / P; the conv bytes stay with
  their compute rank.
* Storage slot of rank r: ceil(N / P) unit positions, then its conv bytes.
  Position i < min(n_r, t_r) holds its own unit i; a deficit position holds
  the unit paired with it; positions >= t_r are not written.
* Send buffer of rank r (one row per checkpoint): its excess units grouped
  by destination rank in increasing order, each group in excess-list order;
  the split sizes are the group sizes.  On load the owners send the units
  back and rank r receives them in the same layout.
* Every unit has the same size (one store): all layers share one unit size.

The functions below follow these steps literally, unit by unit.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .ckpt import pack, unpack_zero_fill
from .plan import GDN, OraclePlan, build_plan


def rank_layers(layers, P: int, r: int):
    """The layer descriptors of rank r's compute-local heads: heads
    [r H / P, (r + 1) H / P) of every layer, with their gate parameters and
    conv_bytes / P."""
    out = []
    for lay in layers:
        assert lay.n_heads % P == 0 and lay.conv_bytes % P == 0
        Hr = lay.n_heads // P
        per = 1 if lay.kind == GDN else lay.d_k
        A = np.asarray(lay.A_log, np.float32).reshape(lay.n_heads, per)[r * Hr:(r + 1) * Hr]
        D = np.asarray(lay.dt_bias, np.float32).reshape(lay.n_heads, per)[r * Hr:(r + 1) * Hr]
        out.append(type(lay)(lay.kind, Hr, lay.d_k, lay.d_v, A.reshape(-1), D.reshape(-1),
                             lay.conv_bytes // P))
    return out


def rank_plans(layers, P: int, a_s: float = -0.3, eps: float = 1e-3, w_max: int = 16):
    """Every rank's own selection plan (its compute-local ragged layout)."""
    return [build_plan(rank_layers(layers, P, r), a_s, eps, w_max) for r in range(P)]


@dataclass
class Balance:
    P: int
    n: list                      # compute-local units per rank
    t: list = field(default_factory=list)       # targets
    keep: list = field(default_factory=list)    # min(n_r, t_r)
    excess: list = field(default_factory=list)  # (source rank, local unit index)
    deficit: list = field(default_factory=list)  # (destination rank, slot position)
    slot_units: int = 0

    @property
    def N(self) -> int:
        return sum(self.n)

    @property
    def M_remote(self) -> int:
        return len(self.excess)

    def dest_of(self, s: int, i: int):
        """Storage owner and slot position of rank s's local unit i."""
        if i < self.keep[s]:
            return s, i
        return self.deficit[self.excess.index((s, i))]

    def send_units(self) -> np.ndarray:
        """[P, P]: units rank s sends to rank d (the all-to-all splits)."""
        M = np.zeros((self.P, self.P), np.int64)
        for (s, _), (d, _) in zip(self.excess, self.deficit):
            M[s, d] += 1
        return M


def storage_balance(n, P: int) -> Balance:
    """[dasc] Appendix B.1(b), step by step."""
    n = [int(x) for x in n]
    assert len(n) == P
    b = Balance(P, n)
    N = sum(n)
    q, m = divmod(N, P)
    order = sorted(range(P), key=lambda r: (-n[r], r))
    t = [0] * P
    for pos, r in enumerate(order):
        t[r] = q + 1 if pos < m else q
    b.t = t
    b.keep = [min(n[r], t[r]) for r in range(P)]
    b.excess = [(r, i) for r in range(P) for i in range(b.keep[r], n[r])]
    b.deficit = [(r, p) for r in range(P) for p in range(b.keep[r], t[r])]
    assert len(b.excess) == len(b.deficit)
    b.slot_units = math.ceil(N / P) if P else 0
    return b


def plans_balance(plans) -> Balance:
    return storage_balance([p.B_temp_rag // _unit_bytes(p) if _unit_bytes(p) else 0
                            for p in plans], len(plans))


def _unit_bytes(plan: OraclePlan) -> int:
    sizes = {lay.unit_bytes for lay in plan.layers}
    assert len(sizes) == 1, "one store: every layer must have the same unit size"
    return sizes.pop()


def slot_bytes_tp(plan: OraclePlan, bal: Balance) -> int:
    return bal.slot_units * _unit_bytes(plan) + plan.B_conv


def send_bytes_tp(plan: OraclePlan, bal: Balance, r: int) -> int:
    return (bal.n[r] - bal.keep[r]) * _unit_bytes(plan)


def _send_position(bal: Balance, s: int, i: int) -> int:
    """Unit index of rank s's excess unit i inside its send row: groups by
    destination rank in increasing order, each in excess-list order."""
    d_i = bal.dest_of(s, i)[0]
    before = 0
    for (s2, i2), (d2, _) in zip(bal.excess, bal.deficit):
        if s2 != s:
            continue
        if d2 < d_i or (d2 == d_i and i2 < i):
            before += 1
    return before


def pack_tp(plan: OraclePlan, bal: Balance, r: int, dense, src_idx, pool, dst_slot, send,
            send_idx) -> None:
    """Store, rank r, before the exchange: pack its compute-local units
    (ragged order), keep units i < keep_r at slot position i, write the
    excess units into the send row, copy its conv bytes after the slot's
    ceil(N / P) unit positions."""
    ub = _unit_bytes(plan)
    conv_at = bal.slot_units * ub
    for si, di, ei in zip(np.asarray(src_idx), np.asarray(dst_slot), np.asarray(send_idx)):
        row = np.zeros((1, plan.slot_bytes), np.uint8)
        pack(plan, dense, [int(si)], row, [0])                 # the rank's ragged units
        for i in range(bal.n[r]):
            unit = row[0, i * ub:(i + 1) * ub]
            if i < bal.keep[r]:
                pool[int(di), i * ub:(i + 1) * ub] = unit
            else:
                j = _send_position(bal, r, i)
                send[int(ei), j * ub:(j + 1) * ub] = unit
        pool[int(di), conv_at:conv_at + plan.B_conv] = row[0, plan.B_temp_rag:plan.slot_bytes]


def exchange_store(plans, bal: Balance, sends, pools, slot) -> None:
    """The variable-split all-to-all of one store, unit by unit: rank s's
    excess unit i, read from its send row sends[s], lands at its paired
    deficit position in the owner's slot pools[d][slot]."""
    for (s, i), (d, p) in zip(bal.excess, bal.deficit):
        ub = _unit_bytes(plans[s])
        j = _send_position(bal, s, i)
        pools[d][slot, p * ub:(p + 1) * ub] = sends[s][j * ub:(j + 1) * ub]


def exchange_load(plans, bal: Balance, pools, slot, recvs) -> None:
    """The inverse transfer of one load: every owner returns the units it
    stores for other ranks; rank s receives them in its send-row layout."""
    for (s, i), (d, p) in zip(bal.excess, bal.deficit):
        ub = _unit_bytes(plans[s])
        j = _send_position(bal, s, i)
        recvs[s][j * ub:(j + 1) * ub] = pools[d][slot, p * ub:(p + 1) * ub]


def unpack_tp(plan: OraclePlan, bal: Balance, r: int, pool, src_slot, recv, recv_idx, dense,
              dst_idx) -> None:
    """Load, rank r, after the inverse exchange: rebuild its ragged units
    (kept units from its slot, the others from the receive row), then unpack
    with zero-fill (dasc-nr, [dasc] §4.2)."""
    ub = _unit_bytes(plan)
    conv_at = bal.slot_units * ub
    for si, ri, di in zip(np.asarray(src_slot), np.asarray(recv_idx), np.asarray(dst_idx)):
        row = np.zeros((1, plan.slot_bytes), np.uint8)
        for i in range(bal.n[r]):
            if i < bal.keep[r]:
                row[0, i * ub:(i + 1) * ub] = pool[int(si), i * ub:(i + 1) * ub]
            else:
                j = _send_position(bal, r, i)
                row[0, i * ub:(i + 1) * ub] = recv[int(ri), j * ub:(j + 1) * ub]
        row[0, plan.B_temp_rag:plan.slot_bytes] = pool[int(si), conv_at:conv_at + plan.B_conv]
        unpack_zero_fill(plan, row, [0], dense, [int(di)])
