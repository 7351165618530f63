/*
 * dasc.h — C ABI of the MI355X (gfx950) state-checkpoint hot path of
 * decay-aware state compression (dasc).
 *
 * Page citations name the page by title and the section / equation there:
 *   [dasc]     "dasc: Decay-Aware State Compression for Hybrid
 *              Linear-Attention Serving" (arXiv HTML version);
 *   [dasc-pp]  the same paper's paperpeel version (Appendix B.2);
 *   [dasc-sum] the picx.dev summary of dasc, "Methodology" (Eq. 6, Eq. 7).
 *
 * Conventions for every call:
 *   - Return value: DASC_OK (0) or a negative DASC_E* code.  A failing call
 *     leaves a message for dasc_last_error() (thread-local) and has not
 *     launched anything.  No C++ exception crosses this boundary.
 *   - Validation is done on the host from host-known sizes only; the host
 *     never reads device memory.  Index arrays that live on the device are
 *     bounds-checked by the kernels themselves: an out-of-range entry is
 *     skipped (no memory outside the given ranges is touched) and sets a
 *     bit in the plan's device status word (dasc_plan_status).
 *   - Data calls (pack, unpack, refresh) are asynchronous on `stream` (a
 *     hipStream_t; NULL is the default stream) and allocate nothing.  The
 *     caller owns every device buffer and keeps it valid until the stream
 *     work completes — in particular a checkpoint being packed stays valid
 *     (and unchanged) until the pack has completed on its stream, which is
 *     the pages' transactional-demotion rule ([dasc-pp] Appendix B.2).
 *   - Device pointers must be 16-byte aligned; strides must be multiples of
 *     16 bytes.  Pool and dense ranges must not overlap.
 *
 * Data layouts (all little-endian, row-major):
 *   dense checkpoint: for each layer l in order, the temporal state
 *     [H_l, d_v, d_k] fp32 with k fastest ([dasc] Appendix E.1 indexes the
 *     state S_{l,h,v,k}); then for each layer in order its conv bytes (bf16,
 *     copied raw).  dense_bytes = sum_l H_l d_v d_k 4 + sum_l conv_bytes_l.
 *   pool slot (ragged Scheme 2, [dasc] Appendix B): for each layer in order,
 *     its r_l retained units in ascending unit order, starting at unit offset
 *     o_l (o_0 = 0, o_{l+1} = o_l + r_l); a GDN unit is one head [d_v, d_k]
 *     fp32, a KDA unit (h, k) is the column S[h, :, k] stored as d_v
 *     contiguous fp32; then every layer's conv bytes (uncompressed,
 *     [dasc-pp] §4.4).  slot_bytes = sum_l r_l unit_bytes_l + sum conv.
 *   units: a GDN unit is a head (index h); a KDA unit is a key channel
 *     (h, k) with index h*d_k + k ([dasc] §4.1).
 *   INT8 pool slot ([dasc] Appendix E.1 Eq. 10 on the ragged layout):
 *     every retained unit's int8 payload, layer by layer in unit order (a
 *     GDN unit as [d_v][d_k] row-major, a KDA unit as its d_v column
 *     entries), padded to 16 bytes; then every retained unit's fp32 scales
 *     in the same order (d_k per GDN unit: one per column k; one per KDA
 *     unit), padded to 16 bytes; then every layer's conv bytes (bf16,
 *     raw).  int8_slot_bytes in dasc_plan_info.
 */
#ifndef DASC_H
#define DASC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DASC_OK 0
#define DASC_EINVAL (-1)        /* bad argument (null, size, alignment, overlap) */
#define DASC_ENOTUPLOADED (-2)  /* data call on a plan whose tables are not on the device */
#define DASC_EHIP (-3)          /* a HIP runtime call failed */
#define DASC_ENOMEM (-4)        /* host allocation failed */
#define DASC_EUNSUPPORTED (-5)  /* shape outside what the kernels implement */

#define DASC_GDN 0  /* head-wise decay: one unit per head */
#define DASC_KDA 1  /* channel-wise decay: one unit per key channel (h, k) */

/* Bits of the device status word. */
#define DASC_STATUS_BAD_INDEX 1u   /* a checkpoint / slot index was out of range */
#define DASC_STATUS_BAD_TOKENS 2u  /* a request's token range was invalid */

typedef struct dasc_plan* dasc_plan_t; /* opaque, library-owned host object */

typedef struct {
  int32_t kind;          /* DASC_GDN or DASC_KDA */
  int32_t n_heads;       /* H_l */
  int32_t d_k;           /* key width (columns of S) */
  int32_t d_v;           /* value width (rows of S) */
  const float* A_log;    /* host; one per unit: [H] (GDN) or [H*d_k] (KDA) */
  const float* dt_bias;  /* host; same shape as A_log */
  int64_t conv_bytes;    /* bf16 conv-state bytes this layer adds (multiple of 16) */
} dasc_layer_desc;

typedef struct {
  int32_t n_layers;
  int32_t w_replay;             /* Eq. 7 window over all local units; 0 if none */
  int64_t n_units;              /* sum_l n_l */
  int64_t n_retained;           /* sum_l r_l */
  int64_t temporal_dense_bytes; /* B_temp^dense */
  int64_t temporal_rag_bytes;   /* B_temp^rag */
  int64_t conv_bytes;           /* B_conv */
  int64_t dense_bytes;          /* bytes of one dense checkpoint */
  int64_t slot_bytes;           /* bytes of one pool slot */
  int64_t r_max;                /* R_max = max_l r_l */
  double r_bar;                 /* mean_l r_l */
  double c_temp;                /* [dasc-sum] Eq. 6: sum n_l / sum r_l (inf if none kept) */
  double c_ckpt;                /* Eq. 6: (B_temp^dense + B_conv) / (B_temp^rag + B_conv) */
  double c_temp_pad;            /* [dasc] App. B Scheme 1: sum n_l / (L R_max) */
  double layout_gain;           /* R_max / r_bar */
  int64_t n_refresh_heads;      /* (layer, head) pairs a refresh replays */
  int64_t device_bytes;         /* size of the device tables (dasc_plan_upload) */
  int64_t k_row, v_row;         /* refresh row widths (elements): sum H d_k, sum H d_v */
  int64_t gate_row, beta_row;   /* sum (H d_k for KDA, H for GDN), sum H */
  int64_t int8_payload_bytes;   /* int8 payload of the retained units */
  int64_t int8_scale_bytes;     /* their fp32 scales */
  int64_t int8_slot_bytes;      /* bytes of one INT8 pool slot (padded blocks + conv) */
  double c_ckpt_int8;           /* dense checkpoint bytes / int8_slot_bytes */
} dasc_plan_info;

typedef struct {
  int32_t kind, n_heads, d_k, d_v;
  int64_t n_units;       /* n_l */
  int64_t n_retained;    /* r_l */
  int64_t unit_offset;   /* o_l (units) */
  int64_t unit_bytes;    /* d_v d_k 4 (GDN) or d_v 4 (KDA) */
  int64_t dense_offset;  /* byte offset of the layer's state in a dense checkpoint */
  int64_t conv_dense_offset;
  int64_t pool_offset;   /* byte offset of the layer's units in a pool slot */
  int64_t conv_pool_offset;
  int64_t conv_bytes;
  int32_t w_layer;       /* max Eq. 7 window over the layer's local units (0 if none) */
  int32_t n_refresh_heads;
  int64_t k_row_offset, v_row_offset, gate_row_offset, beta_row_offset; /* refresh rows */
  int64_t int8_pool_offset;   /* byte offset of the layer's int8 payload in an INT8 slot */
  int64_t int8_scale_offset;  /* ... of its fp32 scales */
} dasc_layer_info;

/* Tensor-parallel storage balancing of one rank ([dasc] §4.3, Appendix
 * B.1(b)); units counted in one store of equal-size units. */
typedef struct {
  int32_t tp, rank;
  int32_t one_store;     /* 1: every layer has the same unit size (balancing available) */
  int32_t reserved;
  int64_t unit_bytes;    /* bytes of one unit */
  int64_t n_total;       /* N = sum_r n_r */
  int64_t slot_units;    /* ceil(N / tp): unit positions of every rank's storage slot */
  int64_t m_remote;      /* units crossing ranks: sum_r max(0, n_r - t_r) */
  int64_t max_local;     /* max_r n_r: the worst rank's units without balancing */
  int64_t n_local;       /* n_r: this rank's compute-local (retained) units */
  int64_t target;        /* t_r */
  int64_t keep;          /* min(n_r, t_r): units this rank keeps, at positions 0 .. keep-1 */
  int64_t send_units;    /* n_r - keep: units this rank stores elsewhere */
  int64_t recv_units;    /* t_r - keep: units it stores for other ranks */
  int64_t slot_bytes;    /* slot_units * unit_bytes + this rank's conv bytes */
  int64_t send_bytes;    /* send_units * unit_bytes: one send / receive row */
} dasc_tp_info;

/*
 * Build the static selection plan ([dasc] §4.1).  For every unit u:
 *   g_u   = -exp(A_log_u) * softplus(a_s + dt_bias_u)      ([dasc] §3.3 Eq. 2)
 *   H_s,u = ln(eps) / g_u                                   ([dasc] §3.3 Eq. 3)
 *   u is retained (global) iff H_s,u > w_max, else local (omitted).
 * Local units get the window W_u = clamp(next_pow2(H_s,u), 4, w_max)
 * ([dasc-sum] Eq. 7).  Computed in double precision on the host.  A gate
 * that underflows to -0 gives H_s = +inf (retained).
 * layers: host array of n_layers descriptors (read during the call only).
 * Requirements: n_heads, d_k, d_v >= 1; d_v*d_k a multiple of 4 (GDN);
 * d_k and d_v multiples of 4 and at most 128 (KDA); conv_bytes >= 0 and a
 * multiple of 16; A_log and dt_bias finite; 0 < eps < 1; w_max >= 0.  The
 * refresh needs d_k == d_v in {16, 32, 64, 128} for every layer it replays
 * (otherwise dasc_ckpt_refresh_suffix returns DASC_EUNSUPPORTED).
 * On success *out owns host memory released by dasc_plan_destroy.
 */
int dasc_plan_build(const dasc_layer_desc* layers, int32_t n_layers, double a_s,
                    double eps, int32_t w_max, dasc_plan_t* out);

/*
 * Plan of one tensor-parallel rank with storage balancing ([dasc] §4.3,
 * Appendix B.1(b)).  `layers` describes the whole model; rank `rank` of `tp`
 * owns heads [rank H/tp, (rank+1) H/tp) of every layer and conv_bytes/tp of
 * each layer's conv state, and the returned plan is the plan_build plan of
 * those heads (its dense checkpoint is the rank's compute-local state;
 * every other call works on it as on any plan).  In addition it holds the
 * storage-balancing map over all tp ranks, from the whole model's
 * selection: with n_r the compute-local retained units of rank r,
 * N = sum n_r and (q, m) = divmod(N, tp), ranks sorted by (-n_r, r) get the
 * targets t_r = q + 1 (first m) or q; rank r keeps its first min(n_r, t_r)
 * units; the excess units (by source rank, then local index) are paired in
 * order with the deficit positions (by destination rank, then position);
 * every rank's storage slot has ceil(N/tp) unit positions.
 * Requirements: 1 <= tp, 0 <= rank < tp, n_heads divisible by tp and
 * conv_bytes by 16 tp for every layer (DASC_EINVAL), and one unit size over
 * all layers (DASC_EUNSUPPORTED).  A plan from dasc_plan_build is rank 0 of 1.
 */
int dasc_plan_build_tp(const dasc_layer_desc* layers, int32_t n_layers, double a_s,
                       double eps, int32_t w_max, int32_t tp, int32_t rank, dasc_plan_t* out);

/* This rank's balancing figures (host only). */
int dasc_plan_tp_info(dasc_plan_t plan, dasc_tp_info* out);

/* The whole map (host only; any pointer may be NULL): send_units[s*tp + d] =
 * units rank s sends to rank d (the variable all-to-all splits), n_local[r]
 * = n_r and target[r] = t_r.  Rank s's send row holds its excess units in
 * its local order, which groups them by destination rank (ascending); rank
 * d receives the group from rank s at slot unit position
 * keep_d + sum_{s' < s} send_units[s'*tp + d].  The load runs the inverse:
 * owners send the same slot ranges back, received in the send-row layout. */
int dasc_plan_tp_splits(dasc_plan_t plan, int64_t* send_units, int64_t* n_local,
                        int64_t* target);

/* Totals and ratios of a plan (host only). */
int dasc_plan_query(dasc_plan_t plan, dasc_plan_info* out);

/* One layer's counts and offsets (host only). */
int dasc_plan_layer(dasc_plan_t plan, int32_t layer, dasc_layer_info* out);

/* Per-unit results for one layer, into caller host arrays of n_l entries
 * (any pointer may be NULL): retained flag (1/0), H_s (double), and the
 * Eq. 7 window W_u for local units (0 for retained units). */
int dasc_plan_units(dasc_plan_t plan, int32_t layer, uint8_t* retained,
                    double* horizon, int32_t* window);

/* [dasc] Appendix C.1 Eq. 8 on one rank: floor(budget / slot_bytes) - 1 slots
 * (slot 0 reserved).  dense != 0 prices a dense slot instead of a pool slot.
 * Returns the count (-1 when the budget holds no slot at all), or INT64_MIN
 * for a null plan or a negative budget. */
int64_t dasc_plan_slots(dasc_plan_t plan, int64_t budget_bytes, int32_t dense);

/* Copy the plan's device tables (task lists, retained-channel masks, gate parameters,
 * status word) into a caller-allocated device buffer of at least
 * info.device_bytes bytes, 256-byte aligned, on `stream`; the copy is
 * complete when this call returns.  Later data calls use that buffer, which
 * must stay valid until the plan is destroyed or uploaded elsewhere.  The
 * status word is cleared. */
int dasc_plan_upload(dasc_plan_t plan, void* device_buffer, int64_t bytes, void* stream);

/* Read (and with clear != 0, then clear) the device status word: an OR of
 * DASC_STATUS_* bits set by kernels since the last clear.  Synchronises
 * `stream`. */
int dasc_plan_status(dasc_plan_t plan, uint32_t* status, int32_t clear, void* stream);

/* Mover calls, for dasc_plan_launches. */
enum {
  DASC_MOVER_PACK = 0,        /* dasc_ckpt_pack */
  DASC_MOVER_UNPACK = 1,      /* dasc_ckpt_unpack_zero_fill */
  DASC_MOVER_PACK_INT8 = 2,   /* dasc_ckpt_pack_int8 */
  DASC_MOVER_UNPACK_INT8 = 3, /* dasc_ckpt_unpack_int8_zero_fill */
  DASC_MOVER_PACK_TP = 4,     /* dasc_ckpt_pack_tp */
  DASC_MOVER_UNPACK_TP = 5    /* dasc_ckpt_unpack_tp_zero_fill */
};

/* How the given mover call over n (checkpoint, slot) pairs is issued: as
 * *launches kernel launches of *pairs_per_launch pairs each (the last may
 * hold fewer).  A call takes launches of a bounded number of pairs, raised
 * where a launch would hold too few workgroups and then evened out; this
 * query lets a caller relate per-launch measurements (profiler traces) to
 * the bytes of its pairs.  Host only; DASC_EINVAL for an unknown mover, a
 * TP mover on a plan that has no TP lists (dasc_plan_tp_info.one_store ==
 * 0), or n < 0. */
int dasc_plan_launches(dasc_plan_t plan, int32_t mover, int32_t n, int32_t* launches,
                       int32_t* pairs_per_launch);

int dasc_plan_destroy(dasc_plan_t plan);

/*
 * Ragged flat-pack, the store path ([dasc] §4.1, Appendix B Scheme 2;
 * [dasc-pp] Appendix B.2 "Insertion and reuse"): for i in [0, n):
 *   pool[dst_slot[i]] <- retained units and conv bytes of dense[src_idx[i]],
 * where dense[j] = dense_base + j*dense_stride (j < n_dense) and pool[s] =
 * pool_base + s*pool_stride (s < n_slots).  Raw bit copies: bit-exact, NaN
 * payloads, -0.0 and denormals preserved.  src_idx / dst_slot: device int32
 * arrays of n entries, in any order; two entries must not name the same
 * destination slot.  Source checkpoints are read only.
 */
int dasc_ckpt_pack(dasc_plan_t plan, const void* dense_base, int64_t dense_stride,
                   int64_t n_dense, const int32_t* src_idx, void* pool_base,
                   int64_t pool_stride, int64_t n_slots, const int32_t* dst_slot,
                   int32_t n, void* stream);

/*
 * Unpack with zero-fill, dasc-nr ([dasc] §4.2): for i in [0, n):
 *   dense[dst_idx[i]] <- the retained units of pool[src_slot[i]] exactly,
 *   +0.0 (all-zero bits) in every local unit, and the stored conv bytes.
 * Every byte of each destination checkpoint is written; the pool is read
 * only (the stored checkpoint is unchanged).  Two entries must not name the
 * same destination checkpoint.
 */
int dasc_ckpt_unpack_zero_fill(dasc_plan_t plan, const void* pool_base,
                               int64_t pool_stride, int64_t n_slots,
                               const int32_t* src_slot, void* dense_base,
                               int64_t dense_stride, int64_t n_dense,
                               const int32_t* dst_idx, int32_t n, void* stream);

/*
 * Bounded-suffix refresh, dasc-wr ([dasc] §4.2): for each request r in
 * [0, n), each layer l and each head h the plan replays (GDN: local heads;
 * KDA: heads with at least one local channel), start from a zero fp32
 * scratch state S [d_v, d_k] and apply, for every token t of the request,
 *   S <- S Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 * ([dasc] §3.1 Eq. 1), where alpha_t = exp(g_t) and g_t = -exp(A_log)
 * softplus(a_t + dt_bias) is the model's gate ([dasc] §3.3 Eq. 2) with the
 * token's own logit a_t (one per head for GDN, per channel for KDA; A_log
 * and dt_bias are the plan's).  Then write only the local units of S into
 * dense[dst_idx[r]]: retained units, the conv bytes and the pool are left
 * untouched.  A request with zero tokens writes zeros into its local units.
 * Arithmetic: fp32 state and gate, bf16 inputs widened exactly.
 * Inputs, token-major over the concatenated tokens of all requests
 * (T = tok_offsets[n] tokens; layer blocks back to back in layer order,
 * heads in order inside a block; per-layer starts in dasc_layer_info):
 *   k     [T, sum_l H_l d_k]  bf16 bits      v    [T, sum_l H_l d_v] bf16 bits
 *   a     [T, sum_l (H_l d_k for KDA, H_l for GDN)] bf16 bits
 *   beta  [T, sum_l H_l]      fp32
 *   k, v and a must be 16-byte aligned; the k and v rows must be multiples
 *   of 8 elements (DASC_EUNSUPPORTED otherwise).
 *   tok_offsets [n+1] int64, device: request r owns tokens
 *     [tok_offsets[r], tok_offsets[r+1]); must be non-decreasing within
 *     [0, n_tokens] (a request that breaks this is skipped and flagged).
 *   n_tokens (= T, the rows of k, v, a and beta) must be below 2^31
 *     (DASC_EINVAL otherwise).
 *   dst_idx [n] int32, device; two entries must not name the same checkpoint.
 */
int dasc_ckpt_refresh_suffix(dasc_plan_t plan, const uint16_t* k, const uint16_t* v,
                             const uint16_t* a, const float* beta,
                             const int64_t* tok_offsets, int64_t n_tokens,
                             void* dense_base, int64_t dense_stride, int64_t n_dense,
                             const int32_t* dst_idx, int32_t n, void* stream);

/*
 * Bounded-suffix refresh, dasc-wr ([dasc] §4.2), with the decays given
 * directly, as Eq. 1 is written ([dasc] §3.1: alpha_t in (0, 1)^{d_k} for
 * KDA, one scalar alpha_t per head for GDN): for each request r in [0, n),
 * each layer l and each head h the plan replays, start from a zero fp32
 * scratch state S [d_v, d_k] and apply, for every token t of the request,
 *   S <- S Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 * then write only the local units of S into dense[dst_idx[r]] (retained
 * units, the conv bytes and the pool are left untouched).  The same call
 * as dasc_ckpt_refresh_suffix except for where the decays come from: the
 * caller's decays, whatever produced them, instead of the plan's gate
 * parameters applied to logits.
 *   alpha [T, sum_l (H_l d_k for KDA, H_l for GDN)] fp32, token-major, the
 *         same row layout as the gate logits of dasc_ckpt_refresh_suffix
 *         (dasc_layer_info.gate_row_offset): KDA head h's decays of token t
 *         at alpha[t][off_l + h d_k + k], a GDN head's at alpha[t][off_l + h].
 *         16-byte aligned.  Values are applied as given (fp32).
 * k, v, beta, tok_offsets, dst_idx, the alignment rules, the arithmetic
 * (fp32 state, bf16 inputs widened exactly) and the errors are those of
 * dasc_ckpt_refresh_suffix.
 */
int dasc_ckpt_refresh_suffix_alpha(dasc_plan_t plan, const uint16_t* k, const uint16_t* v,
                                   const float* alpha, const float* beta,
                                   const int64_t* tok_offsets, int64_t n_tokens,
                                   void* dense_base, int64_t dense_stride, int64_t n_dense,
                                   const int32_t* dst_idx, int32_t n, void* stream);

/*
 * dasc_ckpt_refresh_suffix_alpha with per-head Eq. 7 windows ([dasc-sum]
 * "Methodology" Eq. 7, [dasc] §4.2): head (l, h) of request r replays only
 * the last min(W_lh, n_r) of the request's n_r tokens, W_lh being the
 * largest Eq. 7 window over the head's local units, and writes a head that
 * also holds retained channels as whole rows, as
 * dasc_ckpt_refresh_suffix_windowed does.  Same arguments, rules and errors
 * as dasc_ckpt_refresh_suffix_alpha.
 */
int dasc_ckpt_refresh_suffix_alpha_windowed(dasc_plan_t plan, const uint16_t* k,
                                            const uint16_t* v, const float* alpha,
                                            const float* beta, const int64_t* tok_offsets,
                                            int64_t n_tokens, void* dense_base,
                                            int64_t dense_stride, int64_t n_dense,
                                            const int32_t* dst_idx, int32_t n, void* stream);

/*
 * The same operation as dasc_ckpt_refresh_suffix ([dasc] §3.1 Eq. 1,
 * §4.2), computed in the recurrence's own form: token by token on the
 * vector units (u = S (alpha o k), c = beta (v - u), S <- S Diag(alpha)
 * + c k^T), with the state in registers, instead of in 16-token chunks on
 * the matrix cores.  It exists as the reference point for the chunked form
 * (same inputs, same output, same tolerance against an fp64 replay) and is
 * several times slower.  Same arguments, rules and errors as
 * dasc_ckpt_refresh_suffix.
 */
int dasc_ckpt_refresh_suffix_recurrent(dasc_plan_t plan, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* a, const float* beta,
                                       const int64_t* tok_offsets, int64_t n_tokens,
                                       void* dense_base, int64_t dense_stride, int64_t n_dense,
                                       const int32_t* dst_idx, int32_t n, void* stream);

/*
 * Bounded-suffix refresh with per-head Eq. 7 windows ([dasc-sum]
 * "Methodology" Eq. 7, [dasc] §4.2): as dasc_ckpt_refresh_suffix, except
 * that head (l, h) of request r replays only the last min(W_lh, n_r) of the
 * request's n_r tokens, where W_lh is the largest Eq. 7 window
 * W_u = clamp(next_pow2(H_s,u), 4, w_max) over the head's local units (a
 * KDA head's local channels share one replay because (I - beta k k^T)
 * couples its columns).  The caller passes the suffix for the model-wide
 * window (dasc_plan_info.w_replay, or any longer one); heads whose local
 * units have short horizons then skip the tokens they do not need.  Same
 * arguments, rules and errors as dasc_ckpt_refresh_suffix, with one
 * difference in how the result is written: a replayed KDA head that also
 * holds retained channels is written as whole rows, its retained values read
 * and written back unchanged (a partial write of a 32-byte sector costs the
 * memory a read and a write anyway), so its retained bytes keep their
 * values but no other work may write that head while the call runs.
 */
int dasc_ckpt_refresh_suffix_windowed(dasc_plan_t plan, const uint16_t* k, const uint16_t* v,
                                      const uint16_t* a, const float* beta,
                                      const int64_t* tok_offsets, int64_t n_tokens,
                                      void* dense_base, int64_t dense_stride, int64_t n_dense,
                                      const int32_t* dst_idx, int32_t n, void* stream);

/*
 * Load with refresh in one pass, dasc-wr ([dasc] §4.2): for each request r
 * in [0, n), dense[dst_idx[r]] <- exactly what dasc_ckpt_unpack_zero_fill
 * from pool[src_slot[r]] followed by dasc_ckpt_refresh_suffix (head_windows
 * == 0) or dasc_ckpt_refresh_suffix_windowed (head_windows != 0) over the
 * request's tokens would leave, bit for bit.  Each replayed head is written
 * once, whole: its local columns from the replay and its retained columns
 * from their units in the slot; the other heads and the conv bytes are
 * unpacked as usual.  Arguments as in those two calls (pool rows hold
 * slot_bytes; src_slot and dst_idx: device int32 arrays of n entries).  A
 * request whose token range or indices are invalid is skipped and flagged;
 * its replayed heads are then not written.
 */
int dasc_ckpt_unpack_refresh(dasc_plan_t plan, const void* pool_base, int64_t pool_stride,
                             int64_t n_slots, const int32_t* src_slot, const uint16_t* k,
                             const uint16_t* v, const uint16_t* a, const float* beta,
                             const int64_t* tok_offsets, int64_t n_tokens, void* dense_base,
                             int64_t dense_stride, int64_t n_dense, const int32_t* dst_idx,
                             int32_t n, int32_t head_windows, void* stream);

/*
 * Store with TP storage balancing, this rank's part before the exchange
 * ([dasc] §4.3, Appendix B.1(b): pack and partition): for i in [0, n), the
 * rank's compute-local units of dense[src_idx[i]] in its ragged order
 * (layer by layer, unit by unit) go to
 *   unit j < keep:  pool[dst_slot[i]] at unit position j,
 *   unit j >= keep: send[send_idx[i]] at unit position j - keep,
 * and the rank's conv bytes to pool[dst_slot[i]] at slot_units * unit_bytes.
 * Pool rows hold tp.slot_bytes (pool_stride >= it); unit positions
 * keep .. slot_units-1 are not written (the exchange fills keep .. t_r-1).
 * Send rows hold tp.send_bytes (send_stride >= it, 16-byte aligned) and are
 * ignored (may be NULL) when tp.send_units == 0.  Same rules as
 * dasc_ckpt_pack otherwise; DASC_EUNSUPPORTED if the plan is not one store.
 */
int dasc_ckpt_pack_tp(dasc_plan_t plan, const void* dense_base, int64_t dense_stride,
                      int64_t n_dense, const int32_t* src_idx, void* pool_base,
                      int64_t pool_stride, int64_t n_slots, const int32_t* dst_slot,
                      void* send_base, int64_t send_stride, int64_t n_send,
                      const int32_t* send_idx, int32_t n, void* stream);

/*
 * Load with TP storage balancing, this rank's part after the inverse
 * exchange (gather and zero-fill unpack, dasc-nr, [dasc] §4.2, §4.3): for i
 * in [0, n), dense[dst_idx[i]] <- unit j of the rank's ragged order from
 * pool[src_slot[i]] at position j (j < keep) or from recv[recv_idx[i]] at
 * position j - keep (j >= keep), +0.0 in every local unit, and the conv
 * bytes stored in the slot.  Every byte of each destination is written.
 * Receive rows as the send rows of dasc_ckpt_pack_tp (ignored when
 * tp.send_units == 0).
 */
int dasc_ckpt_unpack_tp_zero_fill(dasc_plan_t plan, const void* pool_base, int64_t pool_stride,
                                  int64_t n_slots, const int32_t* src_slot,
                                  const void* recv_base, int64_t recv_stride, int64_t n_recv,
                                  const int32_t* recv_idx, void* dense_base,
                                  int64_t dense_stride, int64_t n_dense,
                                  const int32_t* dst_idx, int32_t n, void* stream);

/*
 * INT8 pack ([dasc] Appendix E.1 Eq. 10 composed with the ragged layout,
 * §4.1): for i in [0, n), quantize the retained units of dense[src_idx[i]]
 * into INT8 pool slot pool[dst_slot[i]] and copy its conv bytes raw.  Per
 * column k of a retained unit (every column of a GDN head, the one column of
 * a KDA unit), in fp32 with correctly rounded division:
 *   a = max_v |S[v][k]|,  s = max(a, 1e-8) / 127,
 *   q[v] = clip(round_half_even(S[v][k] / s), -127, 127)   (0 if S / s is NaN)
 * Maxima ignore NaN.  Same arguments and rules as dasc_ckpt_pack, except that
 * pool rows hold int8_slot_bytes (pool_stride >= int8_slot_bytes).
 * Requires d_k and d_v multiples of 4 and at most 128 for every layer with
 * a retained unit (DASC_EUNSUPPORTED otherwise).
 */
int dasc_ckpt_pack_int8(dasc_plan_t plan, const void* dense_base, int64_t dense_stride,
                        int64_t n_dense, const int32_t* src_idx, void* pool_base,
                        int64_t pool_stride, int64_t n_slots, const int32_t* dst_slot,
                        int32_t n, void* stream);

/*
 * INT8 unpack with zero-fill, dasc-nr on an INT8 checkpoint ([dasc] §4.2,
 * Appendix E.1): dense[dst_idx[i]] <- S_hat = q s (fp32 product) in every
 * retained unit of pool[src_slot[i]], +0.0 in every local unit, and the
 * stored conv bytes.  Every byte of each destination checkpoint is written;
 * the pool is read only.  Same arguments and rules as
 * dasc_ckpt_unpack_zero_fill with INT8 pool rows.
 */
int dasc_ckpt_unpack_int8_zero_fill(dasc_plan_t plan, const void* pool_base,
                                    int64_t pool_stride, int64_t n_slots,
                                    const int32_t* src_slot, void* dense_base,
                                    int64_t dense_stride, int64_t n_dense,
                                    const int32_t* dst_idx, int32_t n, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* dasc_last_error(void);

/* Library version string. */
const char* dasc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DASC_H */
