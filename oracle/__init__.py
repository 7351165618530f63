"""CPU oracle for the dasc state-checkpoint hot path — TEST INFRASTRUCTURE.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links it, and it imports nothing from the
product path: the two share no code.

Everything here is plain and slow on purpose: NumPy in float64 for floating
point (float32 where the page fixes it: Eq. 10's INT8 quantization), raw bit
copies (uint32 / uint16 views) for data movement, one step of each
definition per line so that it can be checked against the pages by eye.

Pages cited (by title, section / equation / table):

* [dasc]     "dasc: Decay-Aware State Compression for Hybrid Linear-Attention
             Serving" (arXiv HTML version): Eq. 1 (gated delta rule), Eq. 2
             (log-decay gate), Eq. 3 (static horizon), §4.1 (selection mask,
             byte accounting), §4.2 (load policies), Appendix B (padded and
             ragged layouts), Appendix C.1 (Eq. 8, per-rank budgets),
             Appendix E.1 (Eq. 10, INT8), §4.3 and Appendix B.1(b) (TP
             storage balancing).
* [dasc-pp]  the same paper's paperpeel version: Appendix B.2 (insertion and
             reuse, transactional demotion), "Ragged (Scheme 2)".
* [dasc-sum] the picx.dev summary of dasc, "Methodology": the only page that
             prints Eq. 6 (compression ratios) and Eq. 7 (replay window).
* [SEED]     "Shallow Encoding Emits Deep Memories", Appendix B.1 (the same
             recurrence written transposed, and its contraction bound).

Parity pins: every function here is pinned by tests under `tests/` against
closed forms, invariants, printed numbers and brute force (see the
`test_oracle_*` files).  No function is "parity unpinned".
"""
from .plan import (GDN, KDA, OraclePlan, build_plan, gate_log_decay, horizon,
                   next_pow2, replay_window, slots_eq8, softplus)
from .ckpt import pack, unpack_zero_fill
from .int8 import (Int8Layout, dequantize_columns, pack_int8, quantize_columns,
                   unpack_int8_zero_fill)
from .refresh import (bf16_bits_to_f64, delta_rule_step, refresh_expected,
                      replay_dense, replay_rank1)
from .balance import (Balance, exchange_load, exchange_store, pack_tp, plans_balance,
                      rank_layers, rank_plans, send_bytes_tp, slot_bytes_tp, storage_balance,
                      unpack_tp)

__all__ = [
    "GDN", "KDA", "OraclePlan", "build_plan", "gate_log_decay", "horizon",
    "next_pow2", "replay_window", "slots_eq8", "softplus", "pack",
    "unpack_zero_fill", "bf16_bits_to_f64", "delta_rule_step",
    "refresh_expected", "replay_dense", "replay_rank1", "Int8Layout",
    "quantize_columns", "dequantize_columns", "pack_int8", "unpack_int8_zero_fill",
    "Balance", "storage_balance", "plans_balance", "rank_layers", "rank_plans", "pack_tp",
    "unpack_tp", "exchange_store", "exchange_load", "slot_bytes_tp", "send_bytes_tp",
]
