// Internal layouts shared by the host planner and the HIP kernels.
//
// The plan turns the selection mask into flat task lists that the kernels
// walk with one workgroup per (task, checkpoint): no kernel ever decodes the
// mask or the ragged offsets itself.
#pragma once

#include <cstdint>

namespace dasc {

constexpr int kGDN = 0;
constexpr int kKDA = 1;

// Pack and unpack walk one flat list of pieces per direction, in the order
// of the dense checkpoint (layer by layer, head by head, conv last), so that
// the workgroups resident at once sweep a narrow address window.
constexpr uint32_t kPieceCopy = 0;  // move `bytes` between dense and pool
constexpr uint32_t kPieceZero = 1;  // clear `bytes` of the dense checkpoint (unpack)
constexpr uint32_t kPieceKda = 2;   // kKdaRows rows of a KDA head with >= 1 retained channel
// INT8 checkpoints (Eq. 10).  Pack quantizes whole heads (a column's scale
// spans all d_v rows); unpack dequantizes GDN heads kQGdnRows rows at a time
// and KDA heads whole.
constexpr uint32_t kPieceQGdn = 3;  // a retained GDN head
constexpr uint32_t kPieceQKda = 4;  // a KDA head with >= 1 retained channel
// fp32 pack of a d_k = d_v = 128 KDA head: the 32 x 32 block of rows
// kKdaRows rb .. and channels 32 cb .. (cb in the piece's `bytes` field),
// 4 KiB of the dense state, for a block with >= 1 retained channel
constexpr uint32_t kPieceKdaBlock = 5;
// INT8 pack of a d_k = d_v = 128 KDA head with >= 1 retained channel, as
// four 32-channel column blocks of all 128 rows (16 KiB each; a column's
// scale spans the rows, so a block is whole), loaded together and quantized
// in turn by one workgroup; blocks without a retained channel are skipped
constexpr uint32_t kPieceQKdaBlock = 6;
// INT8 pack of a retained d_k = d_v = 128 GDN head, as four 32-column blocks
// loaded together and quantized in turn by one workgroup, which writes the
// head's int8 rows as whole lines
constexpr uint32_t kPieceQGdnBlock = 7;

// Largest byte range one copy / zero piece covers: 256 lanes x 16 B.  Small
// pieces stream HBM markedly faster on MI355X than 64 KiB pieces do.
constexpr uint32_t kCopyChunk = 4096;

// Pairs one mover launch covers: a call over n (checkpoint, slot) pairs is
// issued as launches of at most this many pairs.  Within one launch the
// rate per checkpoint falls as the launch grows (mixed 27-layer model,
// unpack: 5.76 TB/s as eight back-to-back launches of 64 pairs against 5.55
// TB/s as one launch of 512, the same bytes and the same span of time, so
// not a clock or power effect; 5.94-5.96 TB/s at 8-16 pairs); 16 is the
// measured best for the fp32 movers and the INT8 unpack.  A launch also
// keeps at least kMinLaunchGroups workgroups (a TP rank's share of a
// checkpoint has few pieces; short launches pay their start and drain).
// The INT8 pack, one workgroup per 64 KiB head, takes launches of 32 pairs
// and at least kQPackMinGroups workgroups (0.5-1% ahead of 64 pairs and
// 32768 workgroups, and of 16 pairs).
constexpr int kMovePairs = 16;
constexpr int kQPackPairs = 32;
constexpr int64_t kMinLaunchGroups = 32768;
constexpr int64_t kQPackMinGroups = 8192;

// Pairs per launch of a mover call over n pairs of a list of n_pieces
// pieces: at most `per`, raised until a launch holds at least min_groups
// workgroups, then evened out over the launches (64 pairs in launches of 30
// become 22 + 21 + 21, not 30 + 30 + 4).  The number of launches is
// ceil(n / result).  Shared by the launcher and the plan's launch query.
inline int32_t mover_pairs_per_launch(int32_t n, uint32_t n_pieces, int per, int64_t min_groups) {
  if (n <= 0 || n_pieces == 0) return 1;
  const int64_t need = (min_groups + n_pieces - 1) / n_pieces;
  if (need > per) per = need > n ? n : static_cast<int>(need);
  const int32_t launches = (n + per - 1) / per;
  return (n + launches - 1) / launches;
}

// Rows of a KDA head one piece moves: 32 rows make every unit segment a
// whole 128-byte line (32 fp32).
constexpr int kKdaRows = 32;
// LDS floats per staged unit segment (kKdaRows + 4 of padding).
constexpr int kKdaLdsRow = kKdaRows + 4;
// Channels of one KDA block piece (d = 128 heads): 32 rows x 32 channels.
constexpr int kKdaBlockCols = 32;
// Rows of a GDN head one INT8 unpack piece writes: 32 rows of 128 fp32 are
// 16 KiB, four 16-byte stores per lane (unpack pieces of 16 KiB streamed
// HBM best in the fp32 movers).
constexpr int kQGdnRows = 32;

// One workgroup's work for one (checkpoint, slot) pair.  For a KDA piece the
// head's r retained columns (r = popcount of mask) are the units
// pool[pool_off + j d_v 4], j < r, in ascending channel order: channel k
// goes to j = the number of retained channels below k.
struct alignas(64) Piece {
  uint64_t dense_off;  // copy / zero: the range; head pieces: the head's state [d_v][d_k] fp32
  uint64_t pool_off;   // copy: the range; head pieces: the head's first retained unit
  uint32_t type;       // kPiece*
  uint32_t bytes;      // copy / zero: multiple of 16, at most kCopyChunk; KDA block: cb
  uint16_t d_k, d_v;   // head pieces: head shape
  uint16_t rb, r;      // row block (rows kKdaRows rb .., INT8 GDN unpack kQGdnRows rb ..),
                       // retained channels
  uint32_t mask[4];    // KDA: bit k set = channel k retained
  uint64_t scale_off;  // INT8 pieces: byte offset of the first fp32 scale in a slot
  // TP storage balancing (pieces of the pack_tp / unpack_tp lists): units
  // j < split of a KDA piece live in the storage slot at pool_off + j unit;
  // units j >= split live in the rank's send / receive row at
  // alt_off + (j - split) unit.  A copy piece lies wholly on one side:
  // split = 1 (slot, pool_off) or 0 (send / receive row, alt_off).
  uint32_t split;
  uint32_t alt_off;
};

// One (layer, head) that a bounded-suffix refresh replays.
struct alignas(64) RefreshTask {
  uint64_t dense_off;  // the head's state [d][d] in a dense checkpoint
  uint32_t k_off;      // element offset of the head's key in a k row
  uint32_t v_off;      // ... value in a v row
  uint32_t g_off;      // ... gate logit(s) in an `a` row
  uint32_t b_off;      // ... beta in a beta row
  uint32_t param_off;  // index of the head's first unit in the gate arrays
  uint32_t kind;       // kGDN: one gate per head; kKDA: one per channel
  uint32_t local[4];   // bit k set: column k is local and gets written
  uint32_t window;     // Eq. 7 window of the head: max W_u over its local units
  uint32_t pad;
  uint64_t pool_off;   // fused load: byte offset of the head's first retained unit in a slot
};

static_assert(sizeof(Piece) == 64, "Piece layout");
static_assert(sizeof(RefreshTask) == 64, "RefreshTask layout");

// Device pointers of an uploaded plan's sections.
struct DeviceTables {
  const Piece* pack;
  const Piece* unpack;
  const Piece* pack_q;     // INT8 pack
  const Piece* unpack_q;   // INT8 unpack
  const Piece* pack_tp;    // TP storage balancing: pack and partition
  const Piece* unpack_tp;  // ... and the gather of a load
  const Piece* unpack_rest;  // fused load: the unpack pieces of heads no refresh writes
  const RefreshTask* refresh;
  const float* gate_expA;  // exp(A_log) per unit, fp32
  const float* gate_dt;    // dt_bias per unit, fp32
  uint32_t* status;        // DASC_STATUS_* bits
};

// How a refresh task reads its decays: gate logits `a` (bf16, turned into
// decays by Eq. 2 in the kernel) or the decays themselves (fp32 alpha).
constexpr int kGateHead = 0;       // one logit per head (GDN)
constexpr int kGateChan = 1;       // one per channel, 16-byte aligned rows of 8 (KDA)
constexpr int kGateChanSplit = 2;  // one per channel, read element by element (KDA)
constexpr int kGateAlphaHead = 3;       // one fp32 decay per head (GDN)
constexpr int kGateAlphaChan = 4;       // one per channel, 16-byte aligned rows of 8 (KDA)
constexpr int kGateAlphaChanSplit = 5;  // one per channel, read element by element (KDA)
// The decay mode that reads fp32 alpha in place of a logit mode.
constexpr int alpha_gate(int gate) { return gate + kGateAlphaHead; }

constexpr int kRefreshChunk = 16;  // tokens per refresh chunk (the MFMA tile edge)

// A run of refresh tasks that share one kernel instantiation (head width and
// gate mode).
struct Group {
  int32_t d_k, d_v;
  uint32_t first, count;
  int32_t gate;
  uint32_t max_window;  // largest Eq. 7 window of the run's heads
};

// Arguments of one pack or unpack launch: grid x = the pieces, grid y = the
// entry i of the (src_idx[i], dst_idx[i]) pairs.
// pack:   src = dense checkpoints, dst = pool slots
// unpack: src = pool slots,        dst = dense checkpoints
struct MoveArgs {
  const Piece* pieces;
  uint32_t n_pieces;
  int32_t kda_r_max;  // most unit segments a KDA piece stages (sizes the LDS); 0 if none
  bool kda_128;       // every KDA piece has d_k = d_v = 128
  bool q_blocks;      // INT8 pack list of copy pieces and d = 128 block heads only
  const int32_t* src_idx;
  const int32_t* dst_idx;
  const uint8_t* src_base;
  int64_t src_stride, n_src;
  uint8_t* dst_base;
  int64_t dst_stride, n_dst;
  int32_t n;
  uint32_t* status;
  // TP storage-balancing lists (their own kernel instantiation).  Second row
  // per pair for pieces with split < r: the send row (pack) or the receive
  // row (unpack); alt_base == nullptr when no piece uses one.
  bool tp;
  uint8_t* alt_base;
  int64_t alt_stride, n_alt;
  const int32_t* alt_idx;
};

// Kernel launchers (dasc_kernels.hip).  They return a hipError_t value.
int launch_move(bool pack, const MoveArgs& args, void* stream);
// INT8 pack / unpack over an INT8 piece list (kda_r_max and kda_128 unused).
int launch_qmove(bool pack, const MoveArgs& args, void* stream);

bool kda_shape_supported(int d_k, int d_v);
bool refresh_shape_supported(int d_k, int d_v);

struct RefreshArgs {
  const RefreshTask* tasks;
  uint32_t n_tasks;
  const float* gate_expA;
  const float* gate_dt;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* a;      // gate logits (bf16), or
  const float* alpha;     // the decays (fp32), same row layout; non-null selects them
  const float* beta;
  int64_t k_row, v_row, g_row, b_row;
  const int64_t* tok_off;
  int64_t n_tokens;
  uint8_t* dense;
  int64_t dense_stride;
  int64_t n_dense;
  const int32_t* dst_idx;
  int32_t n;
  int32_t head_windows;  // nonzero: each head replays only its last `window` tokens
  int32_t one_chunk;     // with head_windows: every window of the launch is at most one chunk
  uint32_t* status;
  // Fused load (pool != nullptr): request r reads the retained units of
  // slot src_slot[r] and writes each replayed head whole.
  const uint8_t* pool;
  int64_t pool_stride, n_slots;
  const int32_t* src_slot;
};

int launch_refresh(int d, int gate, const RefreshArgs& args, void* stream);
int launch_recurrent(int d, int gate, const RefreshArgs& args, void* stream);

}  // namespace dasc
