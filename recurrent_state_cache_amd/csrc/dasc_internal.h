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

constexpr uint32_t kTaskCopy = 0;  // move `bytes` between dense and pool
constexpr uint32_t kTaskZero = 1;  // clear `bytes` of the dense checkpoint

// Largest byte range one workgroup moves in a copy task (one GDN head at
// d_k = d_v = 128).
constexpr uint32_t kCopyChunk = 65536;

// Bytes of per-head channel maps: ret_list[128] (the r retained channel
// indices, ascending) then rank_of[128] (a channel's position among the
// retained ones, or kLocal).
constexpr uint32_t kMapBytes = 256;
constexpr uint8_t kLocal = 0xFF;

// A contiguous byte range: pack moves dense -> pool, unpack pool -> dense
// (or clears the dense range for kTaskZero).
struct alignas(32) CopyTask {
  uint64_t dense_off;  // byte offset inside a dense checkpoint
  uint64_t pool_off;   // byte offset inside a pool slot
  uint32_t bytes;      // multiple of 16, at most kCopyChunk
  uint32_t type;       // kTaskCopy or kTaskZero
  uint64_t pad;
};

// One KDA head with at least one retained channel.  Its r retained
// columns are the units pool[pool_off + j * d_v * 4], j < r.
struct alignas(32) KdaTask {
  uint64_t dense_off;  // the head's state [d_v][d_k] fp32
  uint64_t pool_off;   // the head's first retained unit
  uint32_t r;          // retained channels of the head
  uint32_t map_idx;    // channel maps at maps + map_idx * kMapBytes
  uint32_t pad[2];
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
  uint32_t pad[4];
};

static_assert(sizeof(CopyTask) == 32, "CopyTask layout");
static_assert(sizeof(KdaTask) == 32, "KdaTask layout");
static_assert(sizeof(RefreshTask) == 64, "RefreshTask layout");

// Device pointers of an uploaded plan's sections.
struct DeviceTables {
  const CopyTask* pack_copy;
  const CopyTask* unpack_copy;
  const KdaTask* kda;
  const uint8_t* maps;
  const RefreshTask* refresh;
  const float* gate_expA;  // exp(A_log) per unit, fp32
  const float* gate_dt;    // dt_bias per unit, fp32
  uint32_t* status;        // DASC_STATUS_* bits
};

// A run of tasks that share one kernel instantiation.  r_max: the largest
// retained-channel count of a KDA head in the run (sizes the LDS).
struct Group {
  int32_t d_k, d_v;
  uint32_t first, count;
  int32_t r_max;
};

// Kernel launchers (dasc_kernels.hip).  They return a hipError_t value.
int launch_copy(bool pack, const CopyTask* tasks, uint32_t n_tasks, const int32_t* src_idx,
                const int32_t* dst_idx, const uint8_t* src_base, int64_t src_stride,
                int64_t n_src, uint8_t* dst_base, int64_t dst_stride, int64_t n_dst,
                int32_t n, uint32_t* status, void* stream);

int launch_kda(bool pack, int d_k, int d_v, int r_max, const KdaTask* tasks, uint32_t n_tasks,
               const uint8_t* maps, const int32_t* src_idx, const int32_t* dst_idx,
               const uint8_t* src_base, int64_t src_stride, int64_t n_src, uint8_t* dst_base,
               int64_t dst_stride, int64_t n_dst, int32_t n, uint32_t* status, void* stream);

bool kda_shape_supported(int d_k, int d_v);
bool refresh_shape_supported(int d_k, int d_v);

struct RefreshArgs {
  const RefreshTask* tasks;
  uint32_t n_tasks;
  const float* gate_expA;
  const float* gate_dt;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* a;
  const float* beta;
  int64_t k_row, v_row, g_row, b_row;
  const int64_t* tok_off;
  int64_t n_tokens;
  uint8_t* dense;
  int64_t dense_stride;
  int64_t n_dense;
  const int32_t* dst_idx;
  int32_t n;
  uint32_t* status;
};

int launch_refresh(int d, const RefreshArgs& args, void* stream);

}  // namespace dasc
