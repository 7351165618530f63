"""The pins must catch plausible mistakes in the oracle.

Each case compiles a copy of one oracle module with one planted mistake (a
dropped term, a wrong sign, a transposed operand, an off-by-one), swaps it
in, and checks that at least one pin test then fails.  CPU only; the real
oracle is restored after every case.
"""
import importlib.util
import inspect
import os
import sys

import pytest

import oracle
import oracle.balance
import oracle.ckpt
import oracle.int8
import oracle.plan
import oracle.refresh
import test_oracle_balance as T_bal
import test_oracle_ckpt as T_ckpt
import test_oracle_int8 as T_int8
import test_oracle_plan as T_plan
import test_oracle_refresh as T_ref

ORACLE_DIR = os.path.dirname(inspect.getfile(oracle))


def _mutant(modname, old, new):
    path = os.path.join(ORACLE_DIR, modname + ".py")
    src = open(path).read()
    assert src.count(old) >= 1, (modname, old)
    src = src.replace(old, new, 1)
    spec = importlib.util.spec_from_loader("oracle._mutant_" + modname, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    sys.modules[spec.name] = mod          # dataclasses look their module up
    exec(compile(src, path + " (mutant)", "exec"), mod.__dict__)
    return mod


def _swap(monkeypatch, modname, mod):
    """Point the oracle package, its submodules and the pin modules at the
    mutant's functions."""
    real = getattr(oracle, modname)
    for name, obj in vars(mod).items():
        if callable(obj) and getattr(real, name, None) is not None and not name.startswith("__"):
            for holder in (oracle, oracle.plan, oracle.ckpt, oracle.refresh, oracle.int8,
                           oracle.balance):
                if getattr(holder, name, None) is getattr(real, name):
                    monkeypatch.setattr(holder, name, obj)


def _some_pin_fails(pins):
    for pin in pins:
        try:
            pin()
        except Exception:
            return True
    return False


PLAN_PINS = [T_plan.test_half_decay_gives_log2_1000, T_plan.test_exact_tie_is_omitted,
             T_plan.test_eq7_windows_worked_by_hand, T_plan.test_gate_inverts_to_chosen_decay,
             T_plan.test_horizon_is_where_decay_reaches_eps,
             T_plan.test_static_logit_lengthens_horizons,
             T_plan.test_ragged_offsets_order_and_bytes,
             T_plan.test_c1_budget_decomposition_and_eq8,
             T_plan.test_eq6_reproduces_kda_2p63_and_eq8_2p64,
             T_plan.test_refreshed_heads_rule, T_plan.test_mask_equals_decay_threshold_rule,
             T_plan.test_head_window_worked_by_hand]
CKPT_PINS = [T_ckpt.test_round_trip_equals_masked_state, T_ckpt.test_pack_is_bijection_onto_payload,
             T_ckpt.test_raw_bits_survive, T_ckpt.test_unpack_overwrites_every_byte_and_zero_is_positive,
             T_ckpt.test_conv_bytes_follow_payload]
REFRESH_PINS = [T_ref.test_rank1_matches_printed_matrix_form, T_ref.test_beta_one_recalls_last_value_exactly,
                T_ref.test_beta_zero_is_pure_column_decay, T_ref.test_one_hot_write_then_decay_closed_form,
                T_ref.test_contraction_bound, lambda: T_ref.test_refresh_expected_wiring_gate_and_rows(8, 8),
                lambda: T_ref.test_refresh_expected_wiring_gate_and_rows(8, 4),
                T_ref.test_refresh_expected_respects_windows, T_ref.test_gdn_scalar_decay_equals_broadcast,
                T_ref.test_head_windows_replay_each_heads_last_tokens,
                lambda: T_ref.test_refresh_expected_alpha_rows(8, 8),
                lambda: T_ref.test_refresh_expected_alpha_rows(4, 12),
                T_ref.test_refresh_expected_alpha_matches_gate_when_alpha_is_the_gate]

INT8_PINS = [T_int8.test_pages_8p11_capacity_and_3p88_quantization_only,
             T_int8.test_scale_is_column_max_over_127_and_rounding_is_half_even,
             T_int8.test_zero_and_tiny_columns_use_the_floor,
             T_int8.test_scales_are_per_key_column_over_values,
             T_int8.test_range_and_error_bound_on_random_columns,
             T_int8.test_non_finite_entries_quantize_to_zero,
             T_int8.test_column_maximum_skips_signaling_nans_in_any_position,
             T_int8.test_pack_unpack_int8_round_trip]

BAL_PINS = [T_bal.test_hand_worked_even_split, T_bal.test_hand_worked_remainder_and_tie_order,
            T_bal.test_indivisible_head_forces_remote_traffic, T_bal.test_target_invariants_random,
            lambda: T_bal.test_store_load_round_trip(T_bal.KDA, 4, 12),
            lambda: T_bal.test_store_load_round_trip(T_bal.GDN, 2, 8),
            T_bal.test_tp1_is_the_plain_ragged_slot, T_bal.test_rank_layers_split_heads_and_parameters]

MUTATIONS = [
    # plan
    ("plan", "np.exp(A_log) * softplus(a + dt_bias)", "np.exp(A_log) * softplus(a - dt_bias)", PLAN_PINS),
    ("plan", "return -np.exp(A_log) * softplus", "return -np.exp(-A_log) * softplus", PLAN_PINS),
    ("plan", "return np.float64(math.log(eps)) / g", "return np.float64(math.log(eps)) * g", PLAN_PINS),
    ("plan", "retained = H > w_max", "retained = H >= w_max", PLAN_PINS),
    ("plan", "while p < x:", "while p <= x:", PLAN_PINS),
    ("plan", "min(max(next_pow2(H_s), 4), w_max)", "max(min(next_pow2(H_s), w_max), 4)", PLAN_PINS),
    ("plan", "p_off += lay.r * lay.unit_bytes", "p_off += lay.n * lay.unit_bytes", PLAN_PINS),
    ("plan", "return np.flatnonzero(~per_head.all(axis=1))", "return np.flatnonzero(~per_head.any(axis=1))", PLAN_PINS),
    ("plan", "c_dense += lay.conv_bytes", "c_dense += 0", PLAN_PINS + CKPT_PINS),
    # pack / unpack
    ("ckpt", "P[j] = S[h, :, k]", "P[j] = S[h, :, (k + 1) % S.shape[2]]", CKPT_PINS),
    ("ckpt", "S[...] = 0", "pass", CKPT_PINS),
    ("ckpt", "S[h, :, k] = P[j]", "S[h, :, (k + 1) % S.shape[2]] = P[j]", CKPT_PINS),
    ("ckpt", "dst[b:b + lay.conv_bytes] = src[a:a + lay.conv_bytes]", "pass", CKPT_PINS),
    # refresh
    ("refresh", 'Ak = np.einsum("...ij,...j->...i", A, k)', 'Ak = np.einsum("...ij,...j->...i", S, k)', REFRESH_PINS),
    ("refresh", "c = beta[..., None] * (v - Ak)", "c = beta[..., None] * (Ak - v)", REFRESH_PINS),
    ("refresh", "c = beta[..., None] * (v - Ak)", "c = (v - Ak)", REFRESH_PINS),
    ("refresh", "A = S * alpha[..., None, :]", "A = S * alpha[..., :, None]", REFRESH_PINS),
    ("refresh", "return A + c[..., :, None] * k[..., None, :]", "return A + k[..., :, None] * c[..., None, :]", REFRESH_PINS),
    ("refresh", "al = np.exp(gate_log_decay(Al, Db, a))", "al = np.exp(-gate_log_decay(Al, Db, a))", REFRESH_PINS),
    ("refresh", "g += lay.n_heads * lay.d_k if lay.kind != GDN else lay.n_heads", "g += lay.n_heads * lay.d_k", REFRESH_PINS),
    ("refresh", "vs = bf16_bits_to_f64(v_bits[t0:t1, vo[li]", "vs = bf16_bits_to_f64(v_bits[t0:t1, ko[li]", REFRESH_PINS),
    ("refresh", "starts = np.maximum(starts, t1 - w)", "starts = np.maximum(starts, t1 - w + 1)", REFRESH_PINS),
    # decays given directly
    ("refresh", "al = alpha[t0:t1, go[li]:go[li] + H].astype(np.float64)[:, hs]", "al = alpha[t0:t1, go[li]:go[li] + H * dk:dk].astype(np.float64)[:, hs]", REFRESH_PINS),
    ("refresh", "al = alpha[t0:t1, go[li]:go[li] + H * dk].astype(np.float64).reshape(-1, H, dk)[:, hs]", "al = alpha[t0:t1, go[li]:go[li] + H * dk].astype(np.float64).reshape(-1, dk, H).transpose(0, 2, 1)[:, hs]", REFRESH_PINS),
    ("refresh", "al = alpha[t0:t1, go[li]:go[li] + H * dk].astype(np.float64).reshape(-1, H, dk)[:, hs]", "al = alpha[t0:t1, ko[li]:ko[li] + H * dk].astype(np.float64).reshape(-1, H, dk)[:, hs]", REFRESH_PINS),
    ("refresh", "al = np.repeat(al[:, :, None], dk, axis=2)                       # alpha_t I", "al = np.repeat(al[:, :1, None], len(hs), axis=1).repeat(dk, axis=2)", REFRESH_PINS),
    ("plan", "return int(lay.W_u[sel].max()) if sel.any() else 0", "return int(lay.W_u[sel].min()) if sel.any() else 0", PLAN_PINS),
    ("plan", "sel = (lay.local_idx // lay.d_k) == h", "sel = (lay.local_idx % lay.d_k) == h", PLAN_PINS),
    # INT8 (Eq. 10)
    ("balance", "key=lambda r: (-n[r], r))", "key=lambda r: (n[r], r))", BAL_PINS),
    ("balance", "key=lambda r: (-n[r], r))", "key=lambda r: (-n[r], -r))", BAL_PINS),
    ("balance", "t[r] = q + 1 if pos < m else q", "t[r] = q + 1 if pos >= P - m else q", BAL_PINS),
    ("balance", "b.keep = [min(n[r], t[r]) for r in range(P)]", "b.keep = [min(n[r], t[r] - 1) if t[r] else 0 for r in range(P)]", BAL_PINS),
    ("balance", "b.excess = [(r, i) for r in range(P) for i in range(b.keep[r], n[r])]", "b.excess = [(r, i) for i in range(max(n + [0])) for r in range(P) if b.keep[r] <= i < n[r]]", BAL_PINS),
    ("balance", "b.slot_units = math.ceil(N / P) if P else 0", "b.slot_units = N // P if P else 0", BAL_PINS),
    ("balance", "if d2 < d_i or (d2 == d_i and i2 < i):", "if d2 > d_i or (d2 == d_i and i2 < i):", BAL_PINS),
    ("balance", "D = np.asarray(lay.dt_bias, np.float32).reshape(lay.n_heads, per)[r * Hr:(r + 1) * Hr]", "D = np.asarray(lay.dt_bias, np.float32).reshape(lay.n_heads, per)[r:r + Hr]", BAL_PINS),
    ("balance", "A = np.asarray(lay.A_log, np.float32).reshape(lay.n_heads, per)[r * Hr:(r + 1) * Hr]", "A = np.asarray(lay.A_log, np.float32).reshape(per, lay.n_heads).T[r * Hr:(r + 1) * Hr]", BAL_PINS),
    ("int8", "s = np.maximum(a, SCALE_FLOOR) / QMAX", "s = np.maximum(a, SCALE_FLOOR) / F32(128.0)", INT8_PINS),
    ("int8", "s = np.maximum(a, SCALE_FLOOR) / QMAX", "s = a / QMAX", INT8_PINS),
    ("int8", "r = np.rint(X / s[None, :])", "r = np.floor(X / s[None, :] + F32(0.5))", INT8_PINS),
    ("int8", "a = np.where(np.isnan(mag), F32(0), mag).max(axis=0)",
     "a = np.full(X.shape[1], np.where(np.isnan(mag), F32(0), mag).max(), F32)", INT8_PINS),
    ("int8", "a = np.where(np.isnan(mag), F32(0), mag).max(axis=0)", "a = np.fmax.reduce(mag, axis=0)",
     INT8_PINS),
    ("int8", "per_unit_s = lay.d_k if lay.kind == GDN else 1", "per_unit_s = 1", INT8_PINS),
    ("int8", "per_unit_q = lay.d_v * lay.d_k if lay.kind == GDN else lay.d_v", "per_unit_q = lay.d_v * lay.d_k", INT8_PINS),
    ("int8", "self.scale_base = align16(q)", "self.scale_base = q", INT8_PINS),
    ("int8", "s = src[so + j * 4:so + (j + 1) * 4].view(F32)", "s = src[so:so + 4].view(F32)", INT8_PINS),
]


@pytest.mark.parametrize("modname,old,new,pins", MUTATIONS,
                         ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_planted_mistake_is_caught(monkeypatch, modname, old, new, pins):
    mod = _mutant(modname, old, new)
    _swap(monkeypatch, modname, mod)
    assert _some_pin_fails(pins), f"no pin caught: {old!r} -> {new!r}"
