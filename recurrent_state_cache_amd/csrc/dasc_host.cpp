// Host side of the dasc checkpoint library: the static selection plan, the
// device task tables, argument validation and the extern "C" entry points.
//
// Pages cited by title:
//   [dasc]     "dasc: Decay-Aware State Compression for Hybrid Linear-Attention
//              Serving" (arXiv HTML version)
//   [dasc-sum] the picx.dev summary of dasc, "Methodology" (Eq. 6, Eq. 7)
//   TP storage balancing: [dasc] §4.3 and Appendix B.1(b).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/dasc.h"
#include "dasc_internal.h"

using namespace dasc;

namespace {

thread_local std::string g_error;

int fail(int code, const std::string& msg) {
  g_error = msg;
  return code;
}

// softplus(x) = ln(1 + e^x), without overflow for large x.
double softplus(double x) {
  return x > 0.0 ? x + std::log1p(std::exp(-x)) : std::log1p(std::exp(x));
}

// Smallest power of two >= x for x > 1; 1 otherwise (NaN included).
double next_pow2(double x) {
  if (!(x > 1.0)) return 1.0;
  double p = 1.0;
  while (p < x) p *= 2.0;
  return p;
}

struct LayerPlan {
  int32_t kind, n_heads, d_k, d_v;
  int64_t n, r;
  int64_t conv_bytes;
  int64_t unit_bytes;
  int64_t unit_off, dense_off, conv_dense_off, pool_off, conv_pool_off;
  int64_t k_row_off, v_row_off, g_row_off, b_row_off;
  int64_t unit_base;  // first unit of the layer in the plan-wide unit order
  int64_t q_off, s_off;  // INT8 slot: payload and scale offsets (bytes, scale block relative)
  int32_t w_layer;
  int32_t n_refresh;
  std::vector<uint8_t> retained;
  std::vector<double> horizon;
  std::vector<int32_t> window;
  std::vector<float> A_log, dt_bias;
};

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

struct dasc_plan {
  std::vector<LayerPlan> layers;
  double a_s = 0, eps = 0;
  int32_t w_max = 0;
  dasc_plan_info info{};
  int64_t k_row = 0, v_row = 0, g_row = 0, b_row = 0;

  // host image of the device tables
  std::vector<Piece> pack, unpack, pack_q, unpack_q, pack_tp, unpack_tp, unpack_rest;
  bool int8_ok = true;          // every layer with a retained unit fits the INT8 kernels
  int64_t int8_scale_base = 0;  // INT8 slot: start of the scale block
  int64_t int8_conv_base = 0;   // INT8 slot: start of the conv bytes
  std::vector<RefreshTask> refresh;
  std::vector<float> gate_expA, gate_dt;
  std::vector<Group> refresh_groups;
  int32_t kda_r_max = 0;  // most unit segments one KDA piece stages
  bool int8_pack_blocks_only = false;  // the INT8 pack list has no whole-head piece
  bool kda_128 = true;    // every KDA layer has d_k = d_v = 128
  int64_t off_pack = 0, off_unpack = 0, off_pack_q = 0, off_unpack_q = 0, off_pack_tp = 0,
          off_unpack_tp = 0, off_unpack_rest = 0, off_refresh = 0, off_expA = 0, off_dt = 0,
          off_status = 0, table_bytes = 0;

  // TP storage balancing of this rank ([dasc] Appendix B.1(b)); a plan from
  // dasc_plan_build is rank 0 of 1 (everything kept).
  dasc_tp_info tp{};
  std::vector<int64_t> tp_counts;  // [tp][tp]: units rank s sends to rank d
  std::vector<int64_t> tp_n, tp_t;  // per rank: compute-local units, target

  uint8_t* device = nullptr;  // caller-owned upload target
  DeviceTables dev{};
};

namespace {

void push_range(std::vector<Piece>& out, uint64_t dense_off, uint64_t pool_off, uint64_t bytes,
                uint32_t type) {
  while (bytes > 0) {
    uint32_t b = static_cast<uint32_t>(std::min<uint64_t>(bytes, kCopyChunk));
    Piece t{};
    t.dense_off = dense_off;
    t.pool_off = pool_off;
    t.bytes = b;
    t.type = type;
    out.push_back(t);
    dense_off += b;
    pool_off += b;
    bytes -= b;
  }
}

// [dasc] Appendix B.1(b): storage targets and the all-to-all splits for
// compute-local unit counts n (one per rank), seen from rank `rank`.
// Returns false if the model is not one store (units of different sizes) or
// a send row would exceed 4 GiB.
bool set_tp(dasc_plan* p, int32_t tp, int32_t rank, const std::vector<int64_t>& n) {
  dasc_tp_info& T = p->tp;
  T = dasc_tp_info{};
  T.tp = tp;
  T.rank = rank;
  int64_t ub = -1;
  bool one = true;
  for (const auto& L : p->layers) {
    if (ub < 0) ub = L.unit_bytes;
    else if (L.unit_bytes != ub) one = false;
  }
  int64_t N = 0, nmax = 0;
  for (int64_t x : n) {
    N += x;
    nmax = std::max(nmax, x);
  }
  const int64_t q = N / tp, m = N % tp;
  std::vector<int32_t> order(tp);
  for (int32_t r = 0; r < tp; ++r) order[r] = r;
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return n[a] != n[b] ? n[a] > n[b] : a < b;  // (-n_r, r)
  });
  p->tp_n = n;
  p->tp_t.assign(tp, q);
  for (int64_t i = 0; i < m; ++i) p->tp_t[order[i]] = q + 1;
  // Pair the excess list (by source rank, then local index) with the deficit
  // list (by destination rank, then position), in order, run by run.
  auto keep = [&](int32_t r) { return std::min(n[r], p->tp_t[r]); };
  std::vector<int64_t> ex(tp), de(tp);
  for (int32_t r = 0; r < tp; ++r) {
    ex[r] = n[r] - keep(r);
    de[r] = p->tp_t[r] - keep(r);
  }
  p->tp_counts.assign(int64_t(tp) * tp, 0);
  int64_t moved = 0;
  for (int32_t s = 0, d = 0;;) {
    while (s < tp && ex[s] == 0) ++s;
    while (d < tp && de[d] == 0) ++d;
    if (s == tp || d == tp) break;
    const int64_t c = std::min(ex[s], de[d]);
    p->tp_counts[int64_t(s) * tp + d] += c;
    ex[s] -= c;
    de[d] -= c;
    moved += c;
  }
  T.one_store = one && ub > 0;
  T.unit_bytes = ub > 0 ? ub : 0;
  T.n_total = N;
  T.slot_units = tp ? (N + tp - 1) / tp : 0;
  T.m_remote = moved;
  T.max_local = nmax;
  T.n_local = n[rank];
  T.target = p->tp_t[rank];
  T.keep = keep(rank);
  T.send_units = n[rank] - T.keep;
  T.recv_units = p->tp_t[rank] - T.keep;
  T.slot_bytes = T.slot_units * T.unit_bytes + p->info.conv_bytes;
  T.send_bytes = T.send_units * T.unit_bytes;
  if (T.send_bytes > int64_t(std::numeric_limits<uint32_t>::max())) T.one_store = 0;
  return T.one_store != 0;
}

// Turn the mask into piece lists and lay out the device tables.  Pieces
// follow the dense checkpoint's order (layers, heads, then conv), which is
// also the pool slot's order.
void build_tables(dasc_plan* p) {
  // The pack list with 32-row pieces for every KDA head: the TP store's list
  // is made from it (on a rank's eighth of the heads the row pieces measured
  // faster than the column blocks).
  std::vector<Piece> pack_rows;
  for (const auto& L : p->layers) {
    int64_t j = 0;  // retained units of the layer seen so far
    if (L.kind == kGDN) {
      for (int h = 0; h < L.n_heads; ++h) {
        const uint64_t d_off = L.dense_off + h * L.unit_bytes;
        if (L.retained[h]) {
          const uint64_t p_off = L.pool_off + j * L.unit_bytes;
          push_range(p->pack, d_off, p_off, L.unit_bytes, kPieceCopy);
          push_range(pack_rows, d_off, p_off, L.unit_bytes, kPieceCopy);
          push_range(p->unpack, d_off, p_off, L.unit_bytes, kPieceCopy);
          ++j;
        } else {
          push_range(p->unpack, d_off, 0, L.unit_bytes, kPieceZero);
        }
      }
      continue;
    }
    p->kda_128 = p->kda_128 && L.d_k == 128 && L.d_v == 128;
    const int64_t head_bytes = int64_t(L.d_v) * L.d_k * 4;
    const int row_blocks = (L.d_v + kKdaRows - 1) / kKdaRows;
    for (int h = 0; h < L.n_heads; ++h) {
      Piece t{};
      uint32_t r = 0;
      for (int k = 0; k < L.d_k; ++k) {
        if (L.retained[h * L.d_k + k]) {
          t.mask[k >> 5] |= 1u << (k & 31);
          ++r;
        }
      }
      const uint64_t d_off = L.dense_off + h * head_bytes;
      if (r == 0) {  // fully omitted head: unpack clears it
        push_range(p->unpack, d_off, 0, head_bytes, kPieceZero);
        continue;
      }
      t.type = kPieceKda;
      t.dense_off = d_off;
      t.pool_off = L.pool_off + j * L.unit_bytes;
      t.d_k = static_cast<uint16_t>(L.d_k);
      t.d_v = static_cast<uint16_t>(L.d_v);
      t.r = static_cast<uint16_t>(r);
      if (L.d_k == 128 && L.d_v == 128) {
        // pack: 32 x 32 blocks (4 KiB) with a retained channel; unpack:
        // 32-row pieces (their contiguous 16 KiB writes measured faster)
        for (int rb = 0; rb < row_blocks; ++rb) {
          Piece u = t;
          u.rb = static_cast<uint16_t>(rb);
          p->unpack.push_back(u);
          pack_rows.push_back(u);
          u.type = kPieceKdaBlock;
          for (uint32_t cb = 0; cb < 128 / kKdaBlockCols; ++cb) {
            u.bytes = cb;
            if (t.mask[cb] != 0) p->pack.push_back(u);
          }
        }
        p->kda_r_max = std::max(p->kda_r_max, static_cast<int32_t>(std::max<uint32_t>(r, kKdaBlockCols)));
      } else {
        for (int rb = 0; rb < row_blocks; ++rb) {
          t.rb = static_cast<uint16_t>(rb);
          p->pack.push_back(t);
          pack_rows.push_back(t);
          p->unpack.push_back(t);
        }
        p->kda_r_max = std::max(p->kda_r_max, static_cast<int32_t>(r));
      }
      j += r;
    }
  }
  // Conv state: one contiguous block after the temporal payload on both sides.
  const dasc_plan_info& I = p->info;
  push_range(p->pack, I.temporal_dense_bytes, I.temporal_rag_bytes, I.conv_bytes, kPieceCopy);
  push_range(pack_rows, I.temporal_dense_bytes, I.temporal_rag_bytes, I.conv_bytes, kPieceCopy);
  push_range(p->unpack, I.temporal_dense_bytes, I.temporal_rag_bytes, I.conv_bytes, kPieceCopy);

  // INT8 pieces ([dasc] Appendix E.1 Eq. 10): pack quantizes each head with a
  // retained unit, d = 128 heads as 32-column blocks (a column's scale spans
  // its rows, so a block holds whole columns) and other heads whole; unpack
  // dequantizes GDN heads by row blocks and KDA heads whole, and clears
  // omitted heads as above.
  // Heads of d = 128 are packed as four 32-column blocks (16 KiB each) that
  // one workgroup loads together and quantizes in turn (kPieceQGdnBlock,
  // kPieceQKdaBlock), writing the head's codes as whole lines.  Measured
  // INT8 pack, GDN workload: 0.61 of the HBM peak as whole heads held in
  // registers (126 VGPRs) with direct stores, 0.48 as one block a workgroup
  // in head order (a head's int8 rows written from four XCDs), 0.63-0.70 as
  // one block a workgroup with a head's four blocks placed on one XCD, 0.71
  // as four blocks a workgroup staged through LDS.
  for (const auto& L : p->layers) {
    const int64_t head_bytes = int64_t(L.d_v) * L.d_k * 4;
    const int row_blocks = (L.d_v + kQGdnRows - 1) / kQGdnRows;
    int64_t j = 0;  // retained units of the layer seen so far
    for (int h = 0; h < L.n_heads; ++h) {
      const uint64_t d_off = L.dense_off + h * head_bytes;
      Piece t{};
      t.dense_off = d_off;
      t.d_k = static_cast<uint16_t>(L.d_k);
      t.d_v = static_cast<uint16_t>(L.d_v);
      uint32_t r = 0;
      if (L.kind == kGDN) {
        r = L.retained[h] ? 1 : 0;
      } else {
        for (int k = 0; k < L.d_k; ++k) {
          if (L.retained[h * L.d_k + k]) {
            t.mask[k >> 5] |= 1u << (k & 31);
            ++r;
          }
        }
      }
      if (r == 0) {
        push_range(p->unpack_q, d_off, 0, head_bytes, kPieceZero);
        continue;
      }
      t.r = static_cast<uint16_t>(r);
      if (L.kind == kGDN) {
        t.type = kPieceQGdn;
        t.pool_off = L.q_off + j * L.d_v * L.d_k;
        t.scale_off = p->int8_scale_base + L.s_off + j * L.d_k * 4;
        Piece b = t;
        if (L.d_k == 128 && L.d_v == 128) b.type = kPieceQGdnBlock;
        p->pack_q.push_back(b);
        for (int rb = 0; rb < row_blocks; ++rb) {
          t.rb = static_cast<uint16_t>(rb);
          p->unpack_q.push_back(t);
        }
      } else {
        t.type = kPieceQKda;
        t.pool_off = L.q_off + j * L.d_v;
        t.scale_off = p->int8_scale_base + L.s_off + j * 4;
        p->unpack_q.push_back(t);
        Piece b = t;
        if (L.d_k == 128 && L.d_v == 128) b.type = kPieceQKdaBlock;
        p->pack_q.push_back(b);
      }
      j += r;
    }
  }
  push_range(p->pack_q, I.temporal_dense_bytes, p->int8_conv_base, I.conv_bytes, kPieceCopy);
  p->int8_pack_blocks_only = std::all_of(p->pack_q.begin(), p->pack_q.end(), [](const Piece& t) {
    return t.type == kPieceCopy || t.type == kPieceQKdaBlock || t.type == kPieceQGdnBlock;
  });
  push_range(p->unpack_q, I.temporal_dense_bytes, p->int8_conv_base, I.conv_bytes, kPieceCopy);

  // TP storage-balancing lists: the fp32 lists with the pool side remapped.
  // Units of the rank's ragged order below keep stay at their slot
  // position; the rest go to the send row in order (the pairing of excess
  // units with deficit positions is monotone, so the send row, grouped by
  // destination rank, is exactly the ragged tail); conv moves behind the
  // slot's slot_units unit positions.
  if (p->tp.one_store) {
    const uint64_t ub = p->tp.unit_bytes, keep = p->tp.keep, keep_b = keep * ub;
    const uint64_t rag = I.temporal_rag_bytes, conv_tp = p->tp.slot_units * ub;
    auto remap = [&](const std::vector<Piece>& in, std::vector<Piece>& out) {
      for (Piece t : in) {
        if (t.type == kPieceZero) {
          out.push_back(t);
        } else if (t.type == kPieceCopy && t.pool_off >= rag) {  // conv bytes
          t.pool_off = t.pool_off - rag + conv_tp;
          t.split = 1;
          out.push_back(t);
        } else if (t.type == kPieceCopy) {  // GDN unit bytes: split at the keep boundary
          const uint64_t a = t.pool_off, b = t.pool_off + t.bytes;
          if (a < keep_b) {
            Piece u = t;
            u.bytes = static_cast<uint32_t>(std::min(b, keep_b) - a);
            u.split = 1;
            out.push_back(u);
          }
          if (b > keep_b) {
            Piece u = t;
            const uint64_t a2 = std::max(a, keep_b);
            u.dense_off = t.dense_off + (a2 - a);
            u.pool_off = a2;
            u.bytes = static_cast<uint32_t>(b - a2);
            u.split = 0;
            u.alt_off = static_cast<uint32_t>(a2 - keep_b);
            out.push_back(u);
          }
        } else {  // KDA piece: units j0 .. j0 + r - 1
          const int64_t j0 = static_cast<int64_t>(t.pool_off / ub);
          const int64_t sp = std::min<int64_t>(std::max<int64_t>(int64_t(keep) - j0, 0), t.r);
          t.split = static_cast<uint32_t>(sp);
          t.alt_off = sp < t.r ? static_cast<uint32_t>((j0 + sp - int64_t(keep)) * ub) : 0u;
          out.push_back(t);
        }
      }
    };
    remap(pack_rows, p->pack_tp);
    remap(p->unpack, p->unpack_tp);
  }

  // Refresh tasks, grouped by head width and gate mode (one kernel each).
  std::vector<std::tuple<int, int, int>> rkeys;  // (d_k, d_v, gate mode)
  std::vector<std::vector<RefreshTask>> rtasks;
  for (const auto& L : p->layers) {
    const int64_t head_bytes = int64_t(L.d_v) * L.d_k * 4;
    int64_t kept = 0;  // retained units of the layer before head h
    for (int h = 0; h < L.n_heads; ++h) {
      RefreshTask t{};
      t.pool_off = static_cast<uint64_t>(L.pool_off + kept * L.unit_bytes);
      if (L.kind == kGDN) {
        kept += L.retained[h];
      } else {
        for (int k = 0; k < L.d_k; ++k) kept += L.retained[int64_t(h) * L.d_k + k];
      }
      bool any_local = false;
      for (int k = 0; k < L.d_k && k < 128; ++k) {
        const int64_t u = L.kind == kGDN ? h : int64_t(h) * L.d_k + k;
        if (!L.retained[u]) {
          t.local[k >> 5] |= 1u << (k & 31);
          t.window = std::max(t.window, static_cast<uint32_t>(L.window[u]));
          any_local = true;
        }
      }
      if (!any_local) continue;
      t.dense_off = L.dense_off + h * head_bytes;
      t.k_off = static_cast<uint32_t>(L.k_row_off + int64_t(h) * L.d_k);
      t.v_off = static_cast<uint32_t>(L.v_row_off + int64_t(h) * L.d_v);
      t.g_off = static_cast<uint32_t>(L.g_row_off + (L.kind == kKDA ? int64_t(h) * L.d_k : h));
      t.b_off = static_cast<uint32_t>(L.b_row_off + h);
      t.param_off = static_cast<uint32_t>(L.unit_base + (L.kind == kKDA ? int64_t(h) * L.d_k : h));
      t.kind = static_cast<uint32_t>(L.kind);
      int gate = kGateHead;
      if (L.kind == kKDA) gate = (t.g_off % 8 == 0 && p->g_row % 8 == 0) ? kGateChan : kGateChanSplit;
      const auto key = std::make_tuple(L.d_k, L.d_v, gate);
      auto it = std::find(rkeys.begin(), rkeys.end(), key);
      if (it == rkeys.end()) {
        rkeys.push_back(key);
        rtasks.emplace_back();
        it = rkeys.end() - 1;
      }
      rtasks[it - rkeys.begin()].push_back(t);
    }
  }
  for (size_t i = 0; i < rkeys.size(); ++i) {
    uint32_t max_window = 0;
    for (const RefreshTask& t : rtasks[i]) max_window = std::max(max_window, t.window);
    Group g{std::get<0>(rkeys[i]), std::get<1>(rkeys[i]), static_cast<uint32_t>(p->refresh.size()),
            static_cast<uint32_t>(rtasks[i].size()), std::get<2>(rkeys[i]), max_window};
    p->refresh.insert(p->refresh.end(), rtasks[i].begin(), rtasks[i].end());
    p->refresh_groups.push_back(g);
  }

  // Fused load: the unpack pieces of every head no refresh task writes (and
  // the conv bytes); pieces never straddle heads.
  {
    std::vector<std::pair<uint64_t, uint64_t>> replayed;  // [start, end) in a dense checkpoint
    for (const auto& L : p->layers) {
      const uint64_t hb = uint64_t(L.d_v) * L.d_k * 4;
      for (const RefreshTask& t : p->refresh)
        if (t.dense_off >= uint64_t(L.dense_off) && t.dense_off < uint64_t(L.dense_off) + L.n_heads * hb)
          replayed.emplace_back(t.dense_off, t.dense_off + hb);
    }
    std::sort(replayed.begin(), replayed.end());
    for (const Piece& t : p->unpack) {
      auto it = std::upper_bound(replayed.begin(), replayed.end(),
                                 std::make_pair(t.dense_off, ~uint64_t(0)));
      const bool inside = it != replayed.begin() && t.dense_off < std::prev(it)->second;
      if (!inside) p->unpack_rest.push_back(t);
    }
  }

  // Gate parameters, per unit in plan order: exp(A_log) rounded once from
  // double, and dt_bias as given.
  for (const auto& L : p->layers) {
    for (int64_t u = 0; u < L.n; ++u) {
      p->gate_expA.push_back(static_cast<float>(std::exp(static_cast<double>(L.A_log[u]))));
      p->gate_dt.push_back(L.dt_bias[u]);
    }
  }

  int64_t o = 0;
  auto section = [&](int64_t bytes) {
    int64_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  p->off_pack = section(p->pack.size() * sizeof(Piece));
  p->off_unpack = section(p->unpack.size() * sizeof(Piece));
  p->off_pack_q = section(p->pack_q.size() * sizeof(Piece));
  p->off_unpack_q = section(p->unpack_q.size() * sizeof(Piece));
  p->off_pack_tp = section(p->pack_tp.size() * sizeof(Piece));
  p->off_unpack_tp = section(p->unpack_tp.size() * sizeof(Piece));
  p->off_unpack_rest = section(p->unpack_rest.size() * sizeof(Piece));
  p->off_refresh = section(p->refresh.size() * sizeof(RefreshTask));
  p->off_expA = section(p->gate_expA.size() * sizeof(float));
  p->off_dt = section(p->gate_dt.size() * sizeof(float));
  p->off_status = section(16);
  p->table_bytes = o;
  p->info.device_bytes = o;
}

}  // namespace

extern "C" {

const char* dasc_last_error(void) { return g_error.c_str(); }

const char* dasc_version(void) { return "dasc-hip 0.1 (gfx950)"; }

static int plan_build_impl(const dasc_layer_desc* layers, int32_t n_layers, double a_s,
                           double eps, int32_t w_max, dasc_plan_t* out) {
  if (!out) return fail(DASC_EINVAL, "plan_build: out is null");
  *out = nullptr;
  if (!layers || n_layers <= 0) return fail(DASC_EINVAL, "plan_build: no layers");
  if (!(eps > 0.0 && eps < 1.0)) return fail(DASC_EINVAL, "plan_build: eps must be in (0, 1)");
  if (w_max < 0) return fail(DASC_EINVAL, "plan_build: w_max must be >= 0");
  if (!std::isfinite(a_s)) return fail(DASC_EINVAL, "plan_build: a_s must be finite");

  dasc_plan* p = new (std::nothrow) dasc_plan();
  if (!p) return fail(DASC_ENOMEM, "plan_build: out of host memory");
  try {
    p->a_s = a_s;
    p->eps = eps;
    p->w_max = w_max;
    const double log_eps = std::log(eps);
    int64_t unit_off = 0, dense_off = 0, pool_off = 0, unit_base = 0;
    int64_t k_row = 0, v_row = 0, g_row = 0, b_row = 0;
    for (int32_t l = 0; l < n_layers; ++l) {
      const dasc_layer_desc& d = layers[l];
      const std::string at = "plan_build: layer " + std::to_string(l) + ": ";
      if (d.kind != kGDN && d.kind != kKDA) {
        delete p;
        return fail(DASC_EINVAL, at + "kind must be DASC_GDN or DASC_KDA");
      }
      if (d.n_heads < 1 || d.d_k < 1 || d.d_v < 1) {
        delete p;
        return fail(DASC_EINVAL, at + "n_heads, d_k and d_v must be >= 1");
      }
      if (d.kind == kGDN && (int64_t(d.d_v) * d.d_k) % 4 != 0) {
        delete p;
        return fail(DASC_EINVAL, at + "GDN head state must be a multiple of 16 bytes");
      }
      if (d.kind == kKDA && !kda_shape_supported(d.d_k, d.d_v)) {
        delete p;
        return fail(DASC_EINVAL, at + "KDA needs d_k and d_v multiples of 4, at most 128");
      }
      if (d.conv_bytes < 0 || d.conv_bytes % 16 != 0) {
        delete p;
        return fail(DASC_EINVAL, at + "conv_bytes must be >= 0 and a multiple of 16");
      }
      if (!d.A_log || !d.dt_bias) {
        delete p;
        return fail(DASC_EINVAL, at + "A_log and dt_bias are required");
      }
      LayerPlan L{};
      L.kind = d.kind;
      L.n_heads = d.n_heads;
      L.d_k = d.d_k;
      L.d_v = d.d_v;
      L.n = d.kind == kGDN ? d.n_heads : int64_t(d.n_heads) * d.d_k;
      L.unit_bytes = d.kind == kGDN ? int64_t(d.d_v) * d.d_k * 4 : int64_t(d.d_v) * 4;
      L.conv_bytes = d.conv_bytes;
      L.A_log.assign(d.A_log, d.A_log + L.n);
      L.dt_bias.assign(d.dt_bias, d.dt_bias + L.n);
      L.retained.resize(L.n);
      L.horizon.resize(L.n);
      L.window.assign(L.n, 0);
      int64_t r = 0;
      int32_t w_layer = 0;
      for (int64_t u = 0; u < L.n; ++u) {
        if (!std::isfinite(L.A_log[u]) || !std::isfinite(L.dt_bias[u])) {
          delete p;
          return fail(DASC_EINVAL, at + "A_log and dt_bias must be finite");
        }
        // [dasc] §3.3 Eq. 2 at the static logit, then Eq. 3.
        const double g = -std::exp(static_cast<double>(L.A_log[u])) *
                         softplus(a_s + static_cast<double>(L.dt_bias[u]));
        const double H = log_eps / g;
        L.horizon[u] = H;
        // [dasc] §4.1: global (retained) iff H_s > W_max.
        const bool keep = H > static_cast<double>(w_max);
        L.retained[u] = keep ? 1 : 0;
        if (keep) {
          ++r;
        } else {
          // [dasc-sum] Eq. 7: clamp(next_pow2(H_s), 4, W_max).
          const double w = std::min(std::max(next_pow2(H), 4.0), static_cast<double>(w_max));
          L.window[u] = static_cast<int32_t>(w);
          w_layer = std::max(w_layer, L.window[u]);
        }
      }
      L.r = r;
      L.w_layer = w_layer;
      L.unit_off = unit_off;
      L.dense_off = dense_off;
      L.pool_off = pool_off;
      L.unit_base = unit_base;
      L.k_row_off = k_row;
      L.v_row_off = v_row;
      L.g_row_off = g_row;
      L.b_row_off = b_row;
      int32_t nref = 0;
      for (int h = 0; h < L.n_heads; ++h) {
        bool any_local = false;
        if (L.kind == kGDN) {
          any_local = !L.retained[h];
        } else {
          for (int k = 0; k < L.d_k; ++k) any_local |= !L.retained[h * L.d_k + k];
        }
        nref += any_local;
      }
      L.n_refresh = nref;
      unit_off += r;
      dense_off += int64_t(L.n_heads) * L.d_v * L.d_k * 4;
      pool_off += r * L.unit_bytes;
      unit_base += L.n;
      k_row += int64_t(L.n_heads) * L.d_k;
      v_row += int64_t(L.n_heads) * L.d_v;
      g_row += L.kind == kKDA ? int64_t(L.n_heads) * L.d_k : L.n_heads;
      b_row += L.n_heads;
      p->layers.push_back(std::move(L));
    }
    // Refresh tasks keep row offsets and gate-parameter indices in 32 bits.
    constexpr int64_t kU32 = std::numeric_limits<uint32_t>::max();
    if (k_row > kU32 || v_row > kU32 || g_row > kU32 || b_row > kU32 || unit_base > kU32) {
      delete p;
      return fail(DASC_EINVAL, "plan_build: model too wide for 32-bit row offsets");
    }
    p->k_row = k_row;
    p->v_row = v_row;
    p->g_row = g_row;
    p->b_row = b_row;
    p->info.k_row = k_row;
    p->info.v_row = v_row;
    p->info.gate_row = g_row;
    p->info.beta_row = b_row;

    dasc_plan_info& I = p->info;
    I.n_layers = n_layers;
    int64_t n_units = 0, n_ret = 0, conv = 0, r_max = 0, nref = 0;
    int32_t w_replay = 0;
    for (auto& L : p->layers) {
      n_units += L.n;
      n_ret += L.r;
      conv += L.conv_bytes;
      r_max = std::max(r_max, L.r);
      w_replay = std::max(w_replay, L.w_layer);
      nref += L.n_refresh;
    }
    I.n_units = n_units;
    I.n_retained = n_ret;
    I.temporal_dense_bytes = dense_off;
    I.temporal_rag_bytes = pool_off;
    I.conv_bytes = conv;
    I.dense_bytes = dense_off + conv;
    I.slot_bytes = pool_off + conv;
    I.r_max = r_max;
    I.w_replay = w_replay;
    I.n_refresh_heads = nref;
    const double inf = std::numeric_limits<double>::infinity();
    I.r_bar = static_cast<double>(n_ret) / n_layers;
    I.c_temp = n_ret ? static_cast<double>(n_units) / static_cast<double>(n_ret) : inf;
    I.c_ckpt = I.slot_bytes ? static_cast<double>(I.dense_bytes) / static_cast<double>(I.slot_bytes) : inf;
    I.c_temp_pad = r_max ? static_cast<double>(n_units) / (static_cast<double>(n_layers) * r_max) : inf;
    I.layout_gain = n_ret ? static_cast<double>(r_max) / I.r_bar : inf;
    int64_t c_dense = dense_off, c_pool = pool_off;
    for (auto& L : p->layers) {
      L.conv_dense_off = c_dense;
      L.conv_pool_off = c_pool;
      c_dense += L.conv_bytes;
      c_pool += L.conv_bytes;
    }
    // INT8 slot ([dasc] Appendix E.1 Eq. 10): int8 payload | fp32 scales |
    // conv, each block 16-byte aligned.
    int64_t q = 0, sc = 0;
    for (auto& L : p->layers) {
      L.q_off = q;
      L.s_off = sc;
      q += L.r * (L.kind == kGDN ? int64_t(L.d_v) * L.d_k : L.d_v);
      sc += L.r * (L.kind == kGDN ? L.d_k : 1) * 4;
      if (L.r > 0 && (L.d_k % 4 || L.d_v % 4 || L.d_k > 128 || L.d_v > 128)) p->int8_ok = false;
    }
    p->int8_scale_base = align_up(q, 16);
    p->int8_conv_base = p->int8_scale_base + align_up(sc, 16);
    I.int8_payload_bytes = q;
    I.int8_scale_bytes = sc;
    I.int8_slot_bytes = p->int8_conv_base + conv;
    I.c_ckpt_int8 = static_cast<double>(I.dense_bytes) / static_cast<double>(I.int8_slot_bytes);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(DASC_ENOMEM, "plan_build: out of host memory");
  }
  *out = p;
  return DASC_OK;
}

static int finish_plan(dasc_plan_t p, int32_t tp, int32_t rank, const std::vector<int64_t>& n,
                       dasc_plan_t* out) {
  try {
    set_tp(p, tp, rank, n);
    build_tables(p);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(DASC_ENOMEM, "plan_build: out of host memory");
  }
  *out = p;
  return DASC_OK;
}

int dasc_plan_build(const dasc_layer_desc* layers, int32_t n_layers, double a_s, double eps,
                    int32_t w_max, dasc_plan_t* out) {
  dasc_plan_t p = nullptr;
  int rc = plan_build_impl(layers, n_layers, a_s, eps, w_max, &p);
  if (rc != DASC_OK) return rc;
  return finish_plan(p, 1, 0, {p->info.n_retained}, out);
}

int dasc_plan_build_tp(const dasc_layer_desc* layers, int32_t n_layers, double a_s, double eps,
                       int32_t w_max, int32_t tp, int32_t rank, dasc_plan_t* out) {
  if (!out) return fail(DASC_EINVAL, "plan_build_tp: out is null");
  *out = nullptr;
  if (tp < 1 || rank < 0 || rank >= tp) return fail(DASC_EINVAL, "plan_build_tp: need 0 <= rank < tp");
  if (!layers || n_layers <= 0) return fail(DASC_EINVAL, "plan_build_tp: no layers");
  for (int32_t l = 0; l < n_layers; ++l)
    if (layers[l].n_heads % tp != 0 || layers[l].conv_bytes % (16 * int64_t(tp)) != 0)
      return fail(DASC_EINVAL, "plan_build_tp: layer " + std::to_string(l) +
                                   ": n_heads must divide by tp and conv_bytes by 16 tp");
  // The whole model's selection gives every rank's compute-local unit count.
  dasc_plan_t full = nullptr;
  int rc = plan_build_impl(layers, n_layers, a_s, eps, w_max, &full);
  if (rc != DASC_OK) return rc;
  std::vector<int64_t> n(tp, 0);
  for (const auto& L : full->layers) {
    const int64_t per = L.kind == kGDN ? 1 : L.d_k, hr = L.n_heads / tp;
    for (int64_t u = 0; u < L.n; ++u) n[(u / per) / hr] += L.retained[u];
  }
  delete full;
  // Rank `rank` owns heads [rank H / tp, (rank + 1) H / tp) of every layer.
  std::vector<dasc_layer_desc> mine(layers, layers + n_layers);
  for (auto& d : mine) {
    const int64_t per = d.kind == kGDN ? 1 : d.d_k;
    d.n_heads /= tp;
    d.A_log += int64_t(rank) * d.n_heads * per;
    d.dt_bias += int64_t(rank) * d.n_heads * per;
    d.conv_bytes /= tp;
  }
  dasc_plan_t p = nullptr;
  rc = plan_build_impl(mine.data(), n_layers, a_s, eps, w_max, &p);
  if (rc != DASC_OK) return rc;
  if (p->info.n_retained != n[rank]) {
    delete p;
    return fail(DASC_EINVAL, "plan_build_tp: inconsistent rank selection");
  }
  rc = finish_plan(p, tp, rank, n, out);
  if (rc != DASC_OK) return rc;
  if (!(*out)->tp.one_store) {
    delete *out;
    *out = nullptr;
    return fail(DASC_EUNSUPPORTED, "plan_build_tp: balancing needs one unit size across layers");
  }
  return DASC_OK;
}

int dasc_plan_tp_info(dasc_plan_t p, dasc_tp_info* out) {
  if (!p || !out) return fail(DASC_EINVAL, "plan_tp_info: null argument");
  *out = p->tp;
  return DASC_OK;
}

int dasc_plan_tp_splits(dasc_plan_t p, int64_t* send_units, int64_t* n_local, int64_t* target) {
  if (!p) return fail(DASC_EINVAL, "plan_tp_splits: null plan");
  const size_t tp = static_cast<size_t>(p->tp.tp);
  if (send_units) std::memcpy(send_units, p->tp_counts.data(), tp * tp * sizeof(int64_t));
  if (n_local) std::memcpy(n_local, p->tp_n.data(), tp * sizeof(int64_t));
  if (target) std::memcpy(target, p->tp_t.data(), tp * sizeof(int64_t));
  return DASC_OK;
}

int dasc_plan_query(dasc_plan_t p, dasc_plan_info* out) {
  if (!p || !out) return fail(DASC_EINVAL, "plan_query: null argument");
  *out = p->info;
  return DASC_OK;
}

int dasc_plan_layer(dasc_plan_t p, int32_t layer, dasc_layer_info* out) {
  if (!p || !out) return fail(DASC_EINVAL, "plan_layer: null argument");
  if (layer < 0 || layer >= static_cast<int32_t>(p->layers.size()))
    return fail(DASC_EINVAL, "plan_layer: layer out of range");
  const LayerPlan& L = p->layers[layer];
  dasc_layer_info I{};
  I.kind = L.kind;
  I.n_heads = L.n_heads;
  I.d_k = L.d_k;
  I.d_v = L.d_v;
  I.n_units = L.n;
  I.n_retained = L.r;
  I.unit_offset = L.unit_off;
  I.unit_bytes = L.unit_bytes;
  I.dense_offset = L.dense_off;
  I.conv_dense_offset = L.conv_dense_off;
  I.pool_offset = L.pool_off;
  I.conv_pool_offset = L.conv_pool_off;
  I.conv_bytes = L.conv_bytes;
  I.w_layer = L.w_layer;
  I.n_refresh_heads = L.n_refresh;
  I.k_row_offset = L.k_row_off;
  I.v_row_offset = L.v_row_off;
  I.gate_row_offset = L.g_row_off;
  I.beta_row_offset = L.b_row_off;
  I.int8_pool_offset = L.q_off;
  I.int8_scale_offset = p->int8_scale_base + L.s_off;
  *out = I;
  return DASC_OK;
}

int dasc_plan_units(dasc_plan_t p, int32_t layer, uint8_t* retained, double* horizon,
                    int32_t* window) {
  if (!p) return fail(DASC_EINVAL, "plan_units: null plan");
  if (layer < 0 || layer >= static_cast<int32_t>(p->layers.size()))
    return fail(DASC_EINVAL, "plan_units: layer out of range");
  const LayerPlan& L = p->layers[layer];
  if (retained) std::memcpy(retained, L.retained.data(), L.n);
  if (horizon) std::memcpy(horizon, L.horizon.data(), L.n * sizeof(double));
  if (window) std::memcpy(window, L.window.data(), L.n * sizeof(int32_t));
  return DASC_OK;
}

int64_t dasc_plan_slots(dasc_plan_t p, int64_t budget_bytes, int32_t dense) {
  if (!p || budget_bytes < 0) {
    fail(DASC_EINVAL, "plan_slots: null plan or negative budget");
    return std::numeric_limits<int64_t>::min();
  }
  const int64_t b = dense ? p->info.dense_bytes : p->info.slot_bytes;
  if (b <= 0) {
    fail(DASC_EINVAL, "plan_slots: empty slot");
    return std::numeric_limits<int64_t>::min();
  }
  // [dasc] Appendix C.1 Eq. 8, one rank: slot 0 is reserved.
  return budget_bytes / b - 1;
}

int dasc_plan_upload(dasc_plan_t p, void* device_buffer, int64_t bytes, void* stream) {
  if (!p || !device_buffer) return fail(DASC_EINVAL, "plan_upload: null argument");
  if (bytes < p->table_bytes) return fail(DASC_EINVAL, "plan_upload: buffer smaller than device_bytes");
  if (reinterpret_cast<uintptr_t>(device_buffer) % 256 != 0)
    return fail(DASC_EINVAL, "plan_upload: buffer must be 256-byte aligned");
  std::vector<uint8_t> img;
  try {
    img.assign(p->table_bytes, 0);
  } catch (const std::bad_alloc&) {
    return fail(DASC_ENOMEM, "plan_upload: out of host memory");
  }
  auto put = [&](int64_t off, const void* src, size_t n) {
    if (n) std::memcpy(img.data() + off, src, n);
  };
  put(p->off_pack, p->pack.data(), p->pack.size() * sizeof(Piece));
  put(p->off_unpack, p->unpack.data(), p->unpack.size() * sizeof(Piece));
  put(p->off_pack_q, p->pack_q.data(), p->pack_q.size() * sizeof(Piece));
  put(p->off_unpack_q, p->unpack_q.data(), p->unpack_q.size() * sizeof(Piece));
  put(p->off_pack_tp, p->pack_tp.data(), p->pack_tp.size() * sizeof(Piece));
  put(p->off_unpack_tp, p->unpack_tp.data(), p->unpack_tp.size() * sizeof(Piece));
  put(p->off_unpack_rest, p->unpack_rest.data(), p->unpack_rest.size() * sizeof(Piece));
  put(p->off_refresh, p->refresh.data(), p->refresh.size() * sizeof(RefreshTask));
  put(p->off_expA, p->gate_expA.data(), p->gate_expA.size() * sizeof(float));
  put(p->off_dt, p->gate_dt.data(), p->gate_dt.size() * sizeof(float));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(device_buffer, img.data(), p->table_bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(DASC_EHIP, std::string("plan_upload: ") + hipGetErrorString(e));
  uint8_t* d = static_cast<uint8_t*>(device_buffer);
  p->device = d;
  p->dev.pack = reinterpret_cast<const Piece*>(d + p->off_pack);
  p->dev.unpack = reinterpret_cast<const Piece*>(d + p->off_unpack);
  p->dev.pack_q = reinterpret_cast<const Piece*>(d + p->off_pack_q);
  p->dev.unpack_q = reinterpret_cast<const Piece*>(d + p->off_unpack_q);
  p->dev.pack_tp = reinterpret_cast<const Piece*>(d + p->off_pack_tp);
  p->dev.unpack_tp = reinterpret_cast<const Piece*>(d + p->off_unpack_tp);
  p->dev.unpack_rest = reinterpret_cast<const Piece*>(d + p->off_unpack_rest);
  p->dev.refresh = reinterpret_cast<const RefreshTask*>(d + p->off_refresh);
  p->dev.gate_expA = reinterpret_cast<const float*>(d + p->off_expA);
  p->dev.gate_dt = reinterpret_cast<const float*>(d + p->off_dt);
  p->dev.status = reinterpret_cast<uint32_t*>(d + p->off_status);
  return DASC_OK;
}

int dasc_plan_status(dasc_plan_t p, uint32_t* status, int32_t clear, void* stream) {
  if (!p || !status) return fail(DASC_EINVAL, "plan_status: null argument");
  if (!p->device) return fail(DASC_ENOTUPLOADED, "plan_status: plan not uploaded");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word[4] = {0, 0, 0, 0};
  hipError_t e = hipMemcpyAsync(word, p->dev.status, sizeof(word), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && clear) {
    const uint32_t zero[4] = {0, 0, 0, 0};
    e = hipMemcpyAsync(p->dev.status, zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
  }
  if (e != hipSuccess) return fail(DASC_EHIP, std::string("plan_status: ") + hipGetErrorString(e));
  *status = word[0];
  return DASC_OK;
}

int dasc_plan_launches(dasc_plan_t p, int32_t mover, int32_t n, int32_t* launches,
                       int32_t* pairs_per_launch) {
  if (!p || !launches || !pairs_per_launch) return fail(DASC_EINVAL, "plan_launches: null argument");
  if (n < 0) return fail(DASC_EINVAL, "plan_launches: n < 0");
  const std::vector<Piece>* list = nullptr;
  int per = kMovePairs;
  int64_t min_groups = kMinLaunchGroups;
  switch (mover) {
    case DASC_MOVER_PACK: list = &p->pack; break;
    case DASC_MOVER_UNPACK: list = &p->unpack; break;
    case DASC_MOVER_PACK_INT8:
      list = &p->pack_q;
      per = kQPackPairs;
      min_groups = kQPackMinGroups;
      break;
    case DASC_MOVER_UNPACK_INT8: list = &p->unpack_q; break;
    case DASC_MOVER_PACK_TP:
    case DASC_MOVER_UNPACK_TP:
      if (!p->tp.one_store) return fail(DASC_EINVAL, "plan_launches: plan has no TP storage balancing");
      list = mover == DASC_MOVER_PACK_TP ? &p->pack_tp : &p->unpack_tp;
      break;
    default: return fail(DASC_EINVAL, "plan_launches: unknown mover");
  }
  const uint32_t np = static_cast<uint32_t>(list->size());
  if (n == 0 || np == 0) {
    *launches = 0;
    *pairs_per_launch = 0;
    return DASC_OK;
  }
  const int32_t pl = mover_pairs_per_launch(n, np, per, min_groups);
  *pairs_per_launch = pl;
  *launches = (n + pl - 1) / pl;
  return DASC_OK;
}

int dasc_plan_destroy(dasc_plan_t p) {
  delete p;
  return DASC_OK;
}

}  // extern "C"

namespace {

bool aligned16(const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; }

bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uintptr_t>(b_bytes) && y < x + static_cast<uintptr_t>(a_bytes);
}

// Common checks of pack and unpack; `what` names the call in messages.
int check_move(const dasc_plan* p, const char* what, const void* dense, int64_t dense_stride,
               int64_t n_dense, const void* pool, int64_t pool_stride, int64_t n_slots,
               const void* idx_a, const void* idx_b, int32_t n, bool int8 = false,
               int64_t slot_override = 0) {
  const std::string w(what);
  if (!p) return fail(DASC_EINVAL, w + ": null plan");
  if (!p->device) return fail(DASC_ENOTUPLOADED, w + ": plan tables not uploaded");
  if (n < 0 || n > 65535) return fail(DASC_EINVAL, w + ": n must be in [0, 65535]");
  if (n == 0) return DASC_OK;
  if (!dense || !pool || !idx_a || !idx_b) return fail(DASC_EINVAL, w + ": null pointer");
  if (!aligned16(dense) || !aligned16(pool)) return fail(DASC_EINVAL, w + ": bases must be 16-byte aligned");
  if (dense_stride < p->info.dense_bytes || dense_stride % 16)
    return fail(DASC_EINVAL, w + ": dense_stride must be >= dense_bytes and a multiple of 16");
  const int64_t slot_bytes = slot_override ? slot_override
                            : int8 ? p->info.int8_slot_bytes : p->info.slot_bytes;
  if (pool_stride < slot_bytes || pool_stride % 16)
    return fail(DASC_EINVAL, w + ": pool_stride must be >= the slot bytes and a multiple of 16");
  if (n_dense <= 0 || n_slots <= 0) return fail(DASC_EINVAL, w + ": n_dense and n_slots must be > 0");
  if (overlap(dense, dense_stride * n_dense, pool, pool_stride * n_slots))
    return fail(DASC_EINVAL, w + ": pool and dense ranges overlap");
  return DASC_OK;
}

// One pack or unpack (fp32 or INT8): a single launch over the direction's
// piece list.
int run_move(const dasc_plan* p, bool pack, const void* src_base, int64_t src_stride,
             int64_t n_src, const int32_t* src_idx, void* dst_base, int64_t dst_stride,
             int64_t n_dst, const int32_t* dst_idx, int32_t n, void* stream, bool int8 = false) {
  const std::vector<Piece>& pieces = int8 ? (pack ? p->pack_q : p->unpack_q)
                                          : (pack ? p->pack : p->unpack);
  MoveArgs m{};
  m.pieces = int8 ? (pack ? p->dev.pack_q : p->dev.unpack_q) : (pack ? p->dev.pack : p->dev.unpack);
  m.n_pieces = static_cast<uint32_t>(pieces.size());
  m.kda_r_max = p->kda_r_max;
  m.kda_128 = p->kda_128;
  m.q_blocks = int8 && pack && p->int8_pack_blocks_only;
  m.src_idx = src_idx;
  m.dst_idx = dst_idx;
  m.src_base = static_cast<const uint8_t*>(src_base);
  m.src_stride = src_stride;
  m.n_src = n_src;
  m.dst_base = static_cast<uint8_t*>(dst_base);
  m.dst_stride = dst_stride;
  m.n_dst = n_dst;
  m.n = n;
  m.status = p->dev.status;
  return int8 ? launch_qmove(pack, m, stream) : launch_move(pack, m, stream);
}

}  // namespace

extern "C" {

int dasc_ckpt_pack(dasc_plan_t p, const void* dense_base, int64_t dense_stride, int64_t n_dense,
                   const int32_t* src_idx, void* pool_base, int64_t pool_stride, int64_t n_slots,
                   const int32_t* dst_slot, int32_t n, void* stream) {
  int rc = check_move(p, "ckpt_pack", dense_base, dense_stride, n_dense, pool_base, pool_stride,
                      n_slots, src_idx, dst_slot, n);
  if (rc != DASC_OK || n == 0) return rc;
  int e = run_move(p, true, dense_base, dense_stride, n_dense, src_idx, pool_base, pool_stride,
                   n_slots, dst_slot, n, stream);
  if (e) return fail(DASC_EHIP, std::string("ckpt_pack: launch failed: ") +
                                    hipGetErrorString(static_cast<hipError_t>(e)));
  return DASC_OK;
}

int dasc_ckpt_unpack_zero_fill(dasc_plan_t p, const void* pool_base, int64_t pool_stride,
                               int64_t n_slots, const int32_t* src_slot, void* dense_base,
                               int64_t dense_stride, int64_t n_dense, const int32_t* dst_idx,
                               int32_t n, void* stream) {
  int rc = check_move(p, "ckpt_unpack_zero_fill", dense_base, dense_stride, n_dense, pool_base,
                      pool_stride, n_slots, src_slot, dst_idx, n);
  if (rc != DASC_OK || n == 0) return rc;
  int e = run_move(p, false, pool_base, pool_stride, n_slots, src_slot, dense_base, dense_stride,
                   n_dense, dst_idx, n, stream);
  if (e) return fail(DASC_EHIP, std::string("ckpt_unpack_zero_fill: launch failed: ") +
                                    hipGetErrorString(static_cast<hipError_t>(e)));
  return DASC_OK;
}

int dasc_ckpt_pack_int8(dasc_plan_t p, const void* dense_base, int64_t dense_stride,
                        int64_t n_dense, const int32_t* src_idx, void* pool_base,
                        int64_t pool_stride, int64_t n_slots, const int32_t* dst_slot, int32_t n,
                        void* stream) {
  int rc = check_move(p, "ckpt_pack_int8", dense_base, dense_stride, n_dense, pool_base,
                      pool_stride, n_slots, src_idx, dst_slot, n, true);
  if (rc != DASC_OK || n == 0) return rc;
  if (!p->int8_ok)
    return fail(DASC_EUNSUPPORTED, "ckpt_pack_int8: INT8 needs d_k, d_v multiples of 4, at most 128");
  int e = run_move(p, true, dense_base, dense_stride, n_dense, src_idx, pool_base, pool_stride,
                   n_slots, dst_slot, n, stream, true);
  if (e) return fail(DASC_EHIP, std::string("ckpt_pack_int8: launch failed: ") +
                                    hipGetErrorString(static_cast<hipError_t>(e)));
  return DASC_OK;
}

int dasc_ckpt_unpack_int8_zero_fill(dasc_plan_t p, const void* pool_base, int64_t pool_stride,
                                    int64_t n_slots, const int32_t* src_slot, void* dense_base,
                                    int64_t dense_stride, int64_t n_dense, const int32_t* dst_idx,
                                    int32_t n, void* stream) {
  int rc = check_move(p, "ckpt_unpack_int8_zero_fill", dense_base, dense_stride, n_dense,
                      pool_base, pool_stride, n_slots, src_slot, dst_idx, n, true);
  if (rc != DASC_OK || n == 0) return rc;
  if (!p->int8_ok)
    return fail(DASC_EUNSUPPORTED,
                "ckpt_unpack_int8_zero_fill: INT8 needs d_k, d_v multiples of 4, at most 128");
  int e = run_move(p, false, pool_base, pool_stride, n_slots, src_slot, dense_base, dense_stride,
                   n_dense, dst_idx, n, stream, true);
  if (e) return fail(DASC_EHIP, std::string("ckpt_unpack_int8_zero_fill: launch failed: ") +
                                    hipGetErrorString(static_cast<hipError_t>(e)));
  return DASC_OK;
}

// TP pack / unpack: the remapped lists, with the send (pack) or receive
// (unpack) rows as the second row of each pair.
static int run_move_tp(const char* w, dasc_plan_t p, bool pack, const void* dense,
                       int64_t dense_stride, int64_t n_dense, const int32_t* dense_idx,
                       const void* pool, int64_t pool_stride, int64_t n_slots,
                       const int32_t* slot_idx, const void* alt, int64_t alt_stride,
                       int64_t n_alt, const int32_t* alt_idx, int32_t n, void* stream) {
  const std::string what(w);
  if (p && !p->tp.one_store)
    return fail(DASC_EUNSUPPORTED, what + ": balancing needs one unit size across layers");
  int rc = check_move(p, w, dense, dense_stride, n_dense, pool, pool_stride, n_slots,
                      dense_idx, slot_idx, n, false, p ? p->tp.slot_bytes : 0);
  if (rc != DASC_OK || n == 0) return rc;
  const bool use_alt = p->tp.send_units > 0;
  if (use_alt) {
    if (!alt || !alt_idx) return fail(DASC_EINVAL, what + ": null send / receive rows");
    if (!aligned16(alt) || alt_stride < p->tp.send_bytes || alt_stride % 16 || n_alt <= 0)
      return fail(DASC_EINVAL, what + ": send / receive rows misaligned or too small");
    if (overlap(alt, alt_stride * n_alt, dense, dense_stride * n_dense) ||
        overlap(alt, alt_stride * n_alt, pool, pool_stride * n_slots))
      return fail(DASC_EINVAL, what + ": send / receive rows overlap dense or pool");
  }
  MoveArgs m{};
  m.pieces = pack ? p->dev.pack_tp : p->dev.unpack_tp;
  m.n_pieces = static_cast<uint32_t>((pack ? p->pack_tp : p->unpack_tp).size());
  m.kda_r_max = p->kda_r_max;
  m.kda_128 = p->kda_128;
  m.src_idx = pack ? dense_idx : slot_idx;
  m.dst_idx = pack ? slot_idx : dense_idx;
  m.src_base = static_cast<const uint8_t*>(pack ? dense : pool);
  m.src_stride = pack ? dense_stride : pool_stride;
  m.n_src = pack ? n_dense : n_slots;
  m.dst_base = static_cast<uint8_t*>(const_cast<void*>(pack ? pool : dense));
  m.dst_stride = pack ? pool_stride : dense_stride;
  m.n_dst = pack ? n_slots : n_dense;
  m.n = n;
  m.status = p->dev.status;
  m.tp = true;
  if (use_alt) {
    m.alt_base = static_cast<uint8_t*>(const_cast<void*>(alt));
    m.alt_stride = alt_stride;
    m.n_alt = n_alt;
    m.alt_idx = alt_idx;
  }
  int e = launch_move(pack, m, stream);
  if (e) return fail(DASC_EHIP, what + ": launch failed: " +
                                    hipGetErrorString(static_cast<hipError_t>(e)));
  return DASC_OK;
}

int dasc_ckpt_pack_tp(dasc_plan_t p, const void* dense_base, int64_t dense_stride,
                      int64_t n_dense, const int32_t* src_idx, void* pool_base,
                      int64_t pool_stride, int64_t n_slots, const int32_t* dst_slot,
                      void* send_base, int64_t send_stride, int64_t n_send,
                      const int32_t* send_idx, int32_t n, void* stream) {
  return run_move_tp("ckpt_pack_tp", p, true, dense_base, dense_stride, n_dense, src_idx,
                     pool_base, pool_stride, n_slots, dst_slot, send_base, send_stride, n_send,
                     send_idx, n, stream);
}

int dasc_ckpt_unpack_tp_zero_fill(dasc_plan_t p, const void* pool_base, int64_t pool_stride,
                                  int64_t n_slots, const int32_t* src_slot,
                                  const void* recv_base, int64_t recv_stride, int64_t n_recv,
                                  const int32_t* recv_idx, void* dense_base,
                                  int64_t dense_stride, int64_t n_dense,
                                  const int32_t* dst_idx, int32_t n, void* stream) {
  return run_move_tp("ckpt_unpack_tp_zero_fill", p, false, dense_base, dense_stride, n_dense,
                     dst_idx, pool_base, pool_stride, n_slots, src_slot, recv_base, recv_stride,
                     n_recv, recv_idx, n, stream);
}

// The refresh in all its forms: `a` (bf16 gate logits) or `alpha` (fp32
// decays) gives the decays, whichever is non-null when the other is null.
static int run_refresh(const char* w, bool head_windows, dasc_plan_t p, const uint16_t* k,
                       const uint16_t* v, const uint16_t* a, const float* beta,
                       const int64_t* tok_offsets, int64_t n_tokens, void* dense_base,
                       int64_t dense_stride, int64_t n_dense, const int32_t* dst_idx, int32_t n,
                       void* stream, const void* pool_base = nullptr, int64_t pool_stride = 0,
                       int64_t n_slots = 0, const int32_t* src_slot = nullptr,
                       bool recurrent = false, const float* alpha = nullptr,
                       bool use_alpha = false) {
  if (!p) return fail(DASC_EINVAL, std::string(w) + ": null plan");
  if (!p->device) return fail(DASC_ENOTUPLOADED, std::string(w) + ": plan tables not uploaded");
  if (n < 0 || n > 65535) return fail(DASC_EINVAL, std::string(w) + ": n must be in [0, 65535]");
  for (const Group& g : p->refresh_groups)
    if (!refresh_shape_supported(g.d_k, g.d_v))
      return fail(DASC_EUNSUPPORTED, std::string(w) + ": refresh needs d_k == d_v in {16, 32, 64, 128}");
  if (n == 0 || p->refresh.empty()) return DASC_OK;
  if (!tok_offsets || !dense_base || !dst_idx) return fail(DASC_EINVAL, std::string(w) + ": null pointer");
  if (n_tokens < 0) return fail(DASC_EINVAL, std::string(w) + ": n_tokens must be >= 0");
  // the kernels index tokens in 32 bits
  if (n_tokens > INT32_MAX) return fail(DASC_EINVAL, std::string(w) + ": n_tokens must be below 2^31");
  const void* decays = use_alpha ? static_cast<const void*>(alpha) : static_cast<const void*>(a);
  if (n_tokens > 0 && (!k || !v || !decays || !beta))
    return fail(DASC_EINVAL, std::string(w) + ": null input pointer");
  if (p->k_row % 8 || p->v_row % 8)
    return fail(DASC_EUNSUPPORTED, std::string(w) + ": k and v rows must be multiples of 8 elements");
  if (n_tokens > 0 && (!aligned16(k) || !aligned16(v) || !aligned16(decays) ||
                       reinterpret_cast<uintptr_t>(beta) % 4))
    return fail(DASC_EINVAL, std::string(w) + (use_alpha ? ": k, v and alpha" : ": k, v and a") +
                                 " must be 16-byte aligned");
  if (!aligned16(dense_base) || dense_stride < p->info.dense_bytes || dense_stride % 16)
    return fail(DASC_EINVAL, std::string(w) + ": dense base/stride misaligned or too small");
  if (n_dense <= 0) return fail(DASC_EINVAL, std::string(w) + ": n_dense must be > 0");
  RefreshArgs args{};
  args.gate_expA = p->dev.gate_expA;
  args.gate_dt = p->dev.gate_dt;
  args.k = k;
  args.v = v;
  args.a = use_alpha ? nullptr : a;
  args.alpha = use_alpha ? alpha : nullptr;
  args.beta = beta;
  args.k_row = p->k_row;
  args.v_row = p->v_row;
  args.g_row = p->g_row;
  args.b_row = p->b_row;
  args.tok_off = tok_offsets;
  args.n_tokens = n_tokens;
  args.dense = static_cast<uint8_t*>(dense_base);
  args.dense_stride = dense_stride;
  args.n_dense = n_dense;
  args.dst_idx = dst_idx;
  args.n = n;
  args.head_windows = head_windows ? 1 : 0;
  args.status = p->dev.status;
  args.pool = static_cast<const uint8_t*>(pool_base);
  args.pool_stride = pool_stride;
  args.n_slots = n_slots;
  args.src_slot = src_slot;
  for (const Group& g : p->refresh_groups) {
    args.tasks = p->dev.refresh + g.first;
    args.n_tasks = g.count;
    args.one_chunk = head_windows && g.max_window <= static_cast<uint32_t>(kRefreshChunk) ? 1 : 0;
    int e = recurrent ? launch_recurrent(g.d_k, g.gate, args, stream)
                      : launch_refresh(g.d_k, g.gate, args, stream);
    if (e) return fail(DASC_EHIP, std::string(w) + ": launch failed: " +
                                      hipGetErrorString(static_cast<hipError_t>(e)));
  }
  return DASC_OK;
}

int dasc_ckpt_refresh_suffix(dasc_plan_t p, const uint16_t* k, const uint16_t* v,
                             const uint16_t* a, const float* beta, const int64_t* tok_offsets,
                             int64_t n_tokens, void* dense_base, int64_t dense_stride,
                             int64_t n_dense, const int32_t* dst_idx, int32_t n, void* stream) {
  return run_refresh("ckpt_refresh_suffix", false, p, k, v, a, beta, tok_offsets, n_tokens,
                     dense_base, dense_stride, n_dense, dst_idx, n, stream);
}

int dasc_ckpt_refresh_suffix_alpha(dasc_plan_t p, const uint16_t* k, const uint16_t* v,
                                   const float* alpha, const float* beta,
                                   const int64_t* tok_offsets, int64_t n_tokens,
                                   void* dense_base, int64_t dense_stride, int64_t n_dense,
                                   const int32_t* dst_idx, int32_t n, void* stream) {
  return run_refresh("ckpt_refresh_suffix_alpha", false, p, k, v, nullptr, beta, tok_offsets,
                     n_tokens, dense_base, dense_stride, n_dense, dst_idx, n, stream, nullptr, 0,
                     0, nullptr, false, alpha, true);
}

int dasc_ckpt_refresh_suffix_alpha_windowed(dasc_plan_t p, const uint16_t* k, const uint16_t* v,
                                            const float* alpha, const float* beta,
                                            const int64_t* tok_offsets, int64_t n_tokens,
                                            void* dense_base, int64_t dense_stride,
                                            int64_t n_dense, const int32_t* dst_idx, int32_t n,
                                            void* stream) {
  return run_refresh("ckpt_refresh_suffix_alpha_windowed", true, p, k, v, nullptr, beta,
                     tok_offsets, n_tokens, dense_base, dense_stride, n_dense, dst_idx, n, stream,
                     nullptr, 0, 0, nullptr, false, alpha, true);
}

int dasc_ckpt_refresh_suffix_recurrent(dasc_plan_t p, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* a, const float* beta,
                                       const int64_t* tok_offsets, int64_t n_tokens,
                                       void* dense_base, int64_t dense_stride, int64_t n_dense,
                                       const int32_t* dst_idx, int32_t n, void* stream) {
  return run_refresh("ckpt_refresh_suffix_recurrent", false, p, k, v, a, beta, tok_offsets,
                     n_tokens, dense_base, dense_stride, n_dense, dst_idx, n, stream, nullptr, 0,
                     0, nullptr, true);
}

int dasc_ckpt_refresh_suffix_windowed(dasc_plan_t p, const uint16_t* k, const uint16_t* v,
                                      const uint16_t* a, const float* beta,
                                      const int64_t* tok_offsets, int64_t n_tokens,
                                      void* dense_base, int64_t dense_stride, int64_t n_dense,
                                      const int32_t* dst_idx, int32_t n, void* stream) {
  return run_refresh("ckpt_refresh_suffix_windowed", true, p, k, v, a, beta, tok_offsets,
                     n_tokens, dense_base, dense_stride, n_dense, dst_idx, n, stream);
}

int dasc_ckpt_unpack_refresh(dasc_plan_t p, const void* pool_base, int64_t pool_stride,
                             int64_t n_slots, const int32_t* src_slot, const uint16_t* k,
                             const uint16_t* v, const uint16_t* a, const float* beta,
                             const int64_t* tok_offsets, int64_t n_tokens, void* dense_base,
                             int64_t dense_stride, int64_t n_dense, const int32_t* dst_idx,
                             int32_t n, int32_t head_windows, void* stream) {
  const char* w = "ckpt_unpack_refresh";
  int rc = check_move(p, w, dense_base, dense_stride, n_dense, pool_base, pool_stride, n_slots,
                      src_slot, dst_idx, n);
  if (rc != DASC_OK || n == 0) return rc;
  // every replayed head, whole (validates the refresh arguments first)
  rc = run_refresh(w, head_windows != 0, p, k, v, a, beta, tok_offsets, n_tokens, dense_base,
                   dense_stride, n_dense, dst_idx, n, stream, pool_base, pool_stride, n_slots,
                   src_slot);
  if (rc != DASC_OK) return rc;
  // heads no refresh task writes, and the conv bytes: the zero-fill unpack
  MoveArgs m{};
  m.pieces = p->dev.unpack_rest;
  m.n_pieces = static_cast<uint32_t>(p->unpack_rest.size());
  m.kda_r_max = p->kda_r_max;
  m.kda_128 = p->kda_128;
  m.src_idx = src_slot;
  m.dst_idx = dst_idx;
  m.src_base = static_cast<const uint8_t*>(pool_base);
  m.src_stride = pool_stride;
  m.n_src = n_slots;
  m.dst_base = static_cast<uint8_t*>(dense_base);
  m.dst_stride = dense_stride;
  m.n_dst = n_dense;
  m.n = n;
  m.status = p->dev.status;
  int e = launch_move(false, m, stream);
  if (e) return fail(DASC_EHIP, std::string(w) + ": launch failed: " +
                                    hipGetErrorString(static_cast<hipError_t>(e)));
  return DASC_OK;
}

}  // extern "C"
