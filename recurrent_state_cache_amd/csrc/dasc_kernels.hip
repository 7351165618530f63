// HIP kernels for gfx950 (CDNA4, wave64) of the dasc checkpoint hot path.
//
// Pages cited by title:
//   [dasc] "dasc: Decay-Aware State Compression for Hybrid Linear-Attention
//          Serving" (arXiv HTML version): §3.1 Eq. 1, §3.3 Eq. 2, §4.1, §4.2,
//          Appendix B (ragged Scheme 2).
//
// Pack and unpack are pure data movement: every workgroup takes one piece of
// the plan's task lists for one (checkpoint, slot) pair and moves raw bits
// with 16-byte accesses.  KDA units are strided columns of a row-major state,
// so a KDA piece (32 rows of a head; for the pack of d = 128 heads a 32 x 32
// column block) goes through registers and LDS.  The refresh keeps one
// head's fp32 state resident in MFMA accumulator registers and replays
// Eq. 1 in exact chunks of 16 tokens.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/dasc.h"
#include "dasc_internal.h"

namespace dasc {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ bool in_range(int64_t i, int64_t n) { return i >= 0 && i < n; }

__device__ __forceinline__ void flag(uint32_t* status, uint32_t bit) { atomicOr(status, bit); }

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void st_stream(T v, T* p) {
  __builtin_nontemporal_store(v, p);
}

// ---------------------------------------------------------------------------
// Pack and unpack ([dasc] §4.1, §4.2, Appendix B Scheme 2).  One launch per
// direction moves every byte of n (checkpoint, slot) pairs: grid x walks the
// plan's piece list (in dense-checkpoint order), grid y the pairs.  Every
// workgroup touches a small, compact range (at most 16 KiB), so that the
// workgroups resident at once sweep a narrow address window; on MI355X that
// streams HBM far better than 64 KiB pieces.  A workgroup issues its three
// table loads (piece, source index, destination index) together, and one
// check consumes all of them, so a piece costs one table round trip before
// its data moves.
//
// Copy / zero pieces: GDN heads (whole units), conv bytes, and the
// zero-fill of omitted GDN heads / fully omitted KDA heads, at most 4 KiB:
// one 16-byte access per lane.
//
// KDA pieces.  The state S is [d_v][d_k] row-major; the unit (h, k) is the
// column S[:, k], stored in the pool as d_v contiguous floats.  A piece is
// one block of kKdaRows = 32 rows of one head: lane (vl, kg) with
// kg = tid % 32, vl = tid / 32 owns the 4x4 block of rows 4 (8 rb + vl) ..
// + 3 and columns 4 kg .. 4 kg + 3, read as four 16-byte row pieces (lanes
// 0..31 of a row cover it contiguously) and transposed in registers.  LDS
// holds only the head's r retained columns, as 32-row segments U[j][..] in
// pool order (j = rank of the channel among the retained ones, a popcount
// of the piece's mask), written and read as 16-byte vectors; each segment
// is one 128-byte line of its unit.  The pack of d = 128 heads uses 32 x 32
// column blocks instead (kda_block_pack below): 4 KiB of reads per
// workgroup, which streams HBM better; the unpack keeps the 32-row pieces,
// whose 16 KiB of contiguous writes measured faster than 8 or 32 KiB.
// ---------------------------------------------------------------------------

// Retained bits of channels 4 kg .. 4 kg + 3 (low 4 bits) and the number of
// retained channels below 4 kg, from a head's 128-bit mask.
// Piece i of a list, read through the constant address space: nothing in a
// launch writes the list, so the words come in as scalar loads (a plain
// load is otherwise made a vector load where the compiler cannot rule out
// the launch's own stores).
__device__ __forceinline__ Piece load_piece(const Piece* list, uint32_t i) {
  using CWords = const __attribute__((address_space(4))) u32x4;
  static_assert(sizeof(Piece) == 4 * sizeof(u32x4), "a piece is four 16-byte words");
  CWords* w = (CWords*)(uintptr_t)list + 4 * static_cast<uint64_t>(i);
  const u32x4 words[4] = {w[0], w[1], w[2], w[3]};
  Piece t;
  __builtin_memcpy(&t, words, sizeof(Piece));
  return t;
}

// Word w (0..3) of a piece's channel mask, selected arithmetically: a chain
// of selects over the four words is otherwise turned into an indexed load,
// which puts a piece held in registers on the stack.
__device__ __forceinline__ uint32_t mask_word(const Piece& t, int w) {
  return (t.mask[0] & (0u - (w == 0))) | (t.mask[1] & (0u - (w == 1))) |
         (t.mask[2] & (0u - (w == 2))) | (t.mask[3] & (0u - (w == 3)));
}

__device__ __forceinline__ void lane_ranks(const Piece& t, int kg, uint32_t& bits4,
                                           uint32_t& below) {
  const int k0 = 4 * kg, w = k0 >> 5, sh = k0 & 31;
  const uint32_t m0 = t.mask[0], m1 = t.mask[1], m2 = t.mask[2], m3 = t.mask[3];
  const uint32_t mw = w == 0 ? m0 : w == 1 ? m1 : w == 2 ? m2 : m3;
  below = (w > 0 ? __popc(m0) : 0u) + (w > 1 ? __popc(m1) : 0u) + (w > 2 ? __popc(m2) : 0u) +
          __popc(mw & ((1u << sh) - 1u));
  bits4 = (mw >> sh) & 0xFu;
}

// Address of unit segment j of a KDA piece on the pool side: the slot row,
// or (TP pieces, j >= split) the send / receive row.
template <bool kAlt>
__device__ __forceinline__ float* unit_seg(const Piece& t, uint8_t* row, uint8_t* alt, int j,
                                           int dv) {
  if constexpr (kAlt) {
    if (j >= static_cast<int>(t.split))
      return reinterpret_cast<float*>(alt + t.alt_off) + (j - static_cast<int>(t.split)) * dv;
  }
  return reinterpret_cast<float*>(row + t.pool_off) + j * dv;
}

template <bool kPack, int DK, int DV, bool kAlt>
__device__ __forceinline__ void kda_piece(const Piece& t, const uint8_t* src, uint8_t* dst,
                                          uint8_t* alt, float* U) {
  const int dk = DK ? DK : t.d_k;
  const int dv = DV ? DV : t.d_v;
  const int KG = dk / 4, VG = dv / 4;
  const int rb = t.rb, r = t.r;
  const int tid = threadIdx.x;
  const int kg = tid % 32, vl = tid / 32, vg = 8 * rb + vl;
  const int nseg = min(8, VG - 8 * rb);  // 16-byte pieces per unit segment
  const bool mine = kg < KG && vl < nseg;
  uint32_t bits4 = 0, below = 0;
  lane_ranks(t, kg, bits4, below);
  if constexpr (kPack) {
    const float* S = reinterpret_cast<const float*>(src + t.dense_off);
    if (mine) {
      f32x4 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[i] = ld_stream(reinterpret_cast<const f32x4*>(S + (4 * vg + i) * dk + 4 * kg));
      uint32_t rk = below;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((bits4 >> c) & 1u) {
          *reinterpret_cast<f32x4*>(&U[rk * kKdaLdsRow + 4 * vl]) =
              f32x4{x[0][c], x[1][c], x[2][c], x[3][c]};
          ++rk;
        }
      }
    }
    __syncthreads();
    for (int q = tid; q < 8 * r; q += kThreads) {
      const int j = q / 8, g = q % 8;
      if (g < nseg)
        st_stream(*reinterpret_cast<const f32x4*>(&U[j * kKdaLdsRow + 4 * g]),
                  reinterpret_cast<f32x4*>(unit_seg<kAlt>(t, dst, alt, j, dv) +
                                           kKdaRows * rb + 4 * g));
    }
  } else {
    for (int q = tid; q < 8 * r; q += kThreads) {
      const int j = q / 8, g = q % 8;
      if (g < nseg)
        *reinterpret_cast<f32x4*>(&U[j * kKdaLdsRow + 4 * g]) =
            ld_stream(reinterpret_cast<const f32x4*>(
                unit_seg<kAlt>(t, const_cast<uint8_t*>(src), alt, j, dv) + kKdaRows * rb +
                4 * g));
    }
    __syncthreads();
    if (mine) {
      float* S = reinterpret_cast<float*>(dst + t.dense_off);
      f32x4 col[4];
      uint32_t rk = below;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((bits4 >> c) & 1u) {
          col[c] = *reinterpret_cast<const f32x4*>(&U[rk * kKdaLdsRow + 4 * vl]);
          ++rk;
        } else {
          col[c] = f32x4{0.f, 0.f, 0.f, 0.f};  // omitted channel: +0.0
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st_stream(f32x4{col[0][i], col[1][i], col[2][i], col[3][i]},
                  reinterpret_cast<f32x4*>(S + (4 * vg + i) * dk + 4 * kg));
    }
  }
}

// KDA block pieces of the pack list (d_k = d_v = 128): the 32 x 32 block of
// rows 32 rb .. and channels 32 cb .. of one head, 4 KiB of the dense
// state, read like a copy piece (workgroups that read 4 KiB stream HBM
// better than 16 KiB ones; blocks without a retained channel are not in the
// list).  Lane (v, cg), v = tid / 8, cg = tid % 8, reads row 32 rb + v,
// channels 32 cb + 4 cg .. + 3 as one 16-byte load (8 lanes cover the
// block's 128-byte row segment) and stores its retained channels into LDS,
// which holds the block's retained columns as 32-row segments (one 128-byte
// line of a unit each); segment j leaves as 16-byte pieces into unit
// (retained channels below 32 cb) + j of the head.  (Unpack keeps the
// 32-row pieces: their contiguous 16 KiB writes measured faster than block
// writes.)
template <bool kAlt>
__device__ __forceinline__ void kda_block_pack(const Piece& t, const uint8_t* src, uint8_t* dst,
                                               uint8_t* alt, float* U) {
  constexpr int D = 128;
  const int cb = static_cast<int>(t.bytes);
  const int tid = threadIdx.x;
  const int v = tid >> 3, cg = tid & 7;
  uint32_t bits4 = 0, below = 0;
  lane_ranks(t, 8 * cb + cg, bits4, below);
  const uint32_t m0 = t.mask[0], m1 = t.mask[1], m2 = t.mask[2];
  const int base = (cb > 0 ? __popc(m0) : 0) + (cb > 1 ? __popc(m1) : 0) + (cb > 2 ? __popc(m2) : 0);
  const uint32_t mc = cb == 0 ? m0 : cb == 1 ? m1 : cb == 2 ? m2 : t.mask[3];
  const int rc = __popc(mc);  // retained channels of the block
  const int row = kKdaRows * t.rb + v;
  const f32x4 x = ld_stream(reinterpret_cast<const f32x4*>(src + t.dense_off) +
                            (row * D + kKdaBlockCols * cb + 4 * cg) / 4);
  uint32_t rk = below - base;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if ((bits4 >> c) & 1u) {
      U[rk * kKdaLdsRow + v] = x[c];
      ++rk;
    }
  }
  __syncthreads();
  const int j = tid >> 3, g = tid & 7;  // segment j, 16-byte piece g
  if (j < rc)
    st_stream(*reinterpret_cast<const f32x4*>(&U[j * kKdaLdsRow + 4 * g]),
              reinterpret_cast<f32x4*>(unit_seg<kAlt>(t, dst, alt, base + j, D) +
                                       kKdaRows * t.rb + 4 * g));
}

template <bool kPack, bool kAlt = false>
__device__ __forceinline__ void copy_piece(const Piece& t, const uint8_t* src, uint8_t* dst,
                                           uint8_t* alt = nullptr) {
  const uint32_t tid = threadIdx.x;
  if (tid >= (t.bytes >> 4)) return;
  uint64_t pool_off = t.pool_off;
  if constexpr (kAlt) {
    if (t.split == 0 && t.type == kPieceCopy) {  // the unit lives in the send / receive row
      pool_off = t.alt_off;
      if (kPack) dst = alt;
      else src = alt;
    }
  }
  const uint64_t src_off = kPack ? t.dense_off : pool_off;
  const uint64_t dst_off = kPack ? pool_off : t.dense_off;
  u32x4* d = reinterpret_cast<u32x4*>(dst + dst_off) + tid;
  if (!kPack && t.type == kPieceZero) {
    st_stream(u32x4{0u, 0u, 0u, 0u}, d);
  } else {
    st_stream(ld_stream(reinterpret_cast<const u32x4*>(src + src_off) + tid), d);
  }
}

// kAlt: the TP storage-balancing lists, whose pieces may address a second
// row per pair (the send row of a pack, the receive row of an unpack).
template <bool kPack, int DK, int DV, bool kAlt>
__global__ void __launch_bounds__(kThreads) move_kernel(MoveArgs a) {
  extern __shared__ __attribute__((aligned(16))) float U[];
  const Piece t = a.pieces[blockIdx.x];
  const int64_t s = a.src_idx[blockIdx.y];
  const int64_t d = a.dst_idx[blockIdx.y];
  const bool has_alt = kAlt && a.alt_base != nullptr;
  const int64_t x = has_alt ? a.alt_idx[blockIdx.y] : 0;
  const bool bad_idx = !in_range(s, a.n_src) || !in_range(d, a.n_dst) ||
                       (has_alt && !in_range(x, a.n_alt));
  const bool block = kPack && t.type == kPieceKdaBlock;
  if (bad_idx | (t.type > kPieceKda && !block)) {
    if (bad_idx && blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, DASC_STATUS_BAD_INDEX);
    return;
  }
  const uint8_t* src = a.src_base + s * a.src_stride;
  uint8_t* dst = a.dst_base + d * a.dst_stride;
  uint8_t* alt = has_alt ? a.alt_base + x * a.alt_stride : nullptr;
  if constexpr (kPack) {
    if (block) {  // uniform per workgroup
      kda_block_pack<kAlt>(t, src, dst, alt, U);
      return;
    }
  }
  if (t.type == kPieceKda)
    kda_piece<kPack, DK, DV, kAlt>(t, src, dst, alt, U);
  else
    copy_piece<kPack, kAlt>(t, src, dst, alt);
}

// ---------------------------------------------------------------------------
// INT8 checkpoints ([dasc] Appendix E.1 Eq. 10) on the ragged layout.  Per
// column k of a retained unit: a = max_v |S[v][k]|, s = max(a, 1e-8) / 127
// and q = clip(round_half_even(S / s), -127, 127), in fp32 with correctly
// rounded division; unpack writes q s (fp32 product).  Maxima are taken with
// `>` so that NaN entries are skipped; a NaN quotient stores 0.
//
// A column's scale spans all d_v rows, so a pack piece holds whole columns.
// d = 128 heads are packed as four 32-column blocks of all rows that one
// workgroup loads together and quantizes in turn (qpack_head_blocks below,
// in an instantiation of its own when the list holds nothing else).  Other
// heads are whole pieces: lane (vl, kg), kg = tid % 32, vl = tid / 32, holds columns
// 4 kg .. 4 kg + 3 of the 16 consecutive rows 16 vl .. 16 vl + 15 in
// registers; the column maxima are combined over the 8 row lanes in LDS.  A
// GDN head writes its int8 rows directly (32 lanes cover a row) and its d_k
// scales.  A KDA head transposes each lane's 16 x 4 int8 block in
// registers, so that a retained column's 16 bytes are one 16-byte LDS store
// into its unit; the units then leave LDS as 16-byte pieces of contiguous
// pool bytes.  Unpack pieces are GDN heads by blocks of 32 rows (lane: 4
// columns of 4 rows, 16 KiB of dense writes per workgroup) and KDA heads
// whole: the units and scales come into LDS as 16-byte pieces, each lane
// reads the 16 bytes of its rows for each of its retained columns and
// writes its 16 rows x 4 columns (+0.0 in omitted columns).  LDS unit rows
// are padded to 144 bytes so that lanes reading or writing different units
// at the same row offset fall on different banks.
// ---------------------------------------------------------------------------
constexpr float kScaleFloor = 1e-8f;
constexpr int kQRows = 16;     // consecutive rows a lane holds (d_v <= 128, 8 row lanes)
constexpr int kQStride = 144;  // bytes per unit row of the LDS staging buffer

// The int8 codes of four entries of four columns.  Eq. 10 rounds the
// correctly rounded fp32 quotient x / s (half to even); the code here comes
// from the product y = x (1 / s), with 1 / s correctly rounded.  Within one
// column |x / s| <= 127 (1 + 2^-23), and y and the
// correctly rounded quotient each lie within a relative 2^-23 + 2^-48 and
// 2^-24 of x / s, so they differ by less than 2.3e-5: their nearest integers
// agree unless y lies within that distance of a half-integer, and only such
// entries (about one in 8000 of random data) take the division.  NaN and
// infinite entries give the same codes on both routes (an infinite column
// maximum makes 1 / s = 0 and every product 0 or NaN, as the quotients are).
constexpr float kHalfGuard = 0.5f - 6e-5f;

//
// The clip of Eq. 10 never binds: every finite entry has |x| at most its
// column's maximum a, so both routes give |x / s| <= 127 (1 + 2^-22) < 127.5
// and a code of magnitude at most 127.  The only entries left to map are
// those with a NaN quotient, which store 0.  The four low bytes are packed
// with byte permutes.
__device__ __forceinline__ uint32_t quant4(f32x4 x, f32x4 s, f32x4 inv) {
  uint32_t q[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float y = x[c] * inv[c];
    float r = rintf(y);
    if (__builtin_expect(fabsf(y - r) > kHalfGuard, 0)) r = rintf(x[c] / s[c]);
    q[c] = r != r ? 0u : static_cast<uint32_t>(static_cast<int32_t>(r));
  }
  // bytes (q0, q1, 0, 0) and (0, 0, q2, q3)
  const uint32_t lo = __builtin_amdgcn_perm(q[1], q[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(q[3], q[2], 0x04000c0cu);
  return lo | hi;
}

// quant4 for the 16 entries of a lane's 4 rows x 4 columns, with one
// branch for the whole set: the products are rounded first, and only if
// any of them lies within the guard of a half-integer are those entries
// redone by division (the same codes as quant4).
__device__ __forceinline__ void quant16(const f32x4 (&x)[4], f32x4 s, f32x4 inv, uint32_t (&w)[4]) {
  float r[4][4];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float y = x[i][c] * inv[c];
      r[i][c] = rintf(y);
      near |= fabsf(y - r[i][c]) > kHalfGuard;
    }
  if (__builtin_expect(near, 0)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (fabsf(x[i][c] * inv[c] - r[i][c]) > kHalfGuard) r[i][c] = rintf(x[i][c] / s[c]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t q[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      q[c] = r[i][c] != r[i][c] ? 0u : static_cast<uint32_t>(static_cast<int32_t>(r[i][c]));
    const uint32_t lo = __builtin_amdgcn_perm(q[1], q[0], 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(q[3], q[2], 0x04000c0cu);
    w[i] = lo | hi;
  }
}

__device__ __forceinline__ f32x4 dequant4(uint32_t w, f32x4 s) {
  f32x4 x;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    x[c] = static_cast<float>(static_cast<int8_t>((w >> (8 * c)) & 0xFFu)) * s[c];
  return x;
}

// 4 x 4 byte transpose: byte c of a[i] becomes byte i of b[c].
__device__ __forceinline__ void transpose4(const uint32_t (&a)[4], uint32_t (&b)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) x |= ((a[i] >> (8 * c)) & 0xFFu) << (8 * i);
    b[c] = x;
  }
}

__device__ __forceinline__ float load_scale(const uint8_t* p) {
  return *reinterpret_cast<const float*>(p);
}

// Pack of a GDN head: every unit of the head, whole.
__device__ __forceinline__ void qpack_gdn_head(const Piece& t, const uint8_t* src, uint8_t* dst,
                                               float (&red)[8][128]) {
  const int dk = t.d_k, dv = t.d_v, KG = dk / 4;
  const int tid = threadIdx.x, kg = tid % 32, vl = tid / 32;
  const bool col_on = kg < KG;
  const float* S = reinterpret_cast<const float*>(src + t.dense_off);
  f32x4 x[kQRows];
  f32x4 mx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kQRows; ++i) {
    const int v = kQRows * vl + i;
    x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (col_on && v < dv) {
      x[i] = ld_stream(reinterpret_cast<const f32x4*>(S + v * dk + 4 * kg));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float m = fabsf(x[i][c]);
        mx[c] = m > mx[c] ? m : mx[c];
      }
    }
  }
  *reinterpret_cast<f32x4*>(&red[vl][4 * kg]) = mx;
  __syncthreads();
  if (!col_on) return;
  f32x4 sc, inv;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) m = red[r][4 * kg + c] > m ? red[r][4 * kg + c] : m;
    sc[c] = (m > kScaleFloor ? m : kScaleFloor) / 127.f;  // correctly rounded fp32 division
    inv[c] = 1.f / sc[c];
  }
  uint8_t* Q = dst + t.pool_off;
#pragma unroll
  for (int i = 0; i < kQRows; ++i) {
    const int v = kQRows * vl + i;
    if (v < dv) *reinterpret_cast<uint32_t*>(Q + v * dk + 4 * kg) = quant4(x[i], sc, inv);
  }
  if (vl == 0) {
    float* Sc = reinterpret_cast<float*>(dst + t.scale_off);
#pragma unroll
    for (int c = 0; c < 4; ++c) Sc[4 * kg + c] = sc[c];
  }
}

// Pack of a KDA head with a retained channel, whole: lane (vl, kg) as for
// a GDN head; each retained column's bytes of the lane's 16 rows go to its
// unit in LDS as one 16-byte store, then the head's units leave LDS as
// 16-byte pieces of contiguous pool bytes.
__device__ __forceinline__ void qpack_kda_head(const Piece& t, const uint8_t* src, uint8_t* dst,
                                               float (&red)[8][128], uint8_t* qbuf) {
  const int dk = t.d_k, dv = t.d_v, KG = dk / 4;
  const int tid = threadIdx.x, kg = tid % 32, vl = tid / 32;
  const bool col_on = kg < KG;
  uint32_t bits4 = 0, below = 0;
  lane_ranks(t, kg, bits4, below);
  const float* S = reinterpret_cast<const float*>(src + t.dense_off);
  f32x4 x[kQRows];
  f32x4 mx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kQRows; ++i) {
    const int v = kQRows * vl + i;
    x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (col_on && v < dv) {
      x[i] = ld_stream(reinterpret_cast<const f32x4*>(S + v * dk + 4 * kg));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float m = fabsf(x[i][c]);
        mx[c] = m > mx[c] ? m : mx[c];
      }
    }
  }
  *reinterpret_cast<f32x4*>(&red[vl][4 * kg]) = mx;
  __syncthreads();
  if (col_on) {
    f32x4 sc, inv;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) m = red[r][4 * kg + c] > m ? red[r][4 * kg + c] : m;
      sc[c] = (m > kScaleFloor ? m : kScaleFloor) / 127.f;  // correctly rounded fp32 division
      inv[c] = 1.f / sc[c];
    }
    uint32_t cw[4][4];  // [column c][row group m]; rows >= d_v hold zeros, never copied out
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w[4] = {quant4(x[4 * m], sc, inv), quant4(x[4 * m + 1], sc, inv),
                             quant4(x[4 * m + 2], sc, inv), quant4(x[4 * m + 3], sc, inv)};
      uint32_t b[4];
      transpose4(w, b);
#pragma unroll
      for (int c = 0; c < 4; ++c) cw[c][m] = b[c];
    }
    uint32_t rk = below;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((bits4 >> c) & 1u) {
        *reinterpret_cast<u32x4*>(&qbuf[rk * kQStride + 16 * vl]) =
            u32x4{cw[c][0], cw[c][1], cw[c][2], cw[c][3]};
        ++rk;
      }
    }
    if (vl == 0) {
      float* Sc = reinterpret_cast<float*>(dst + t.scale_off);
      rk = below;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((bits4 >> c) & 1u) {
          Sc[rk] = sc[c];
          ++rk;
        }
      }
    }
  }
  __syncthreads();
  const int r = t.r;
  uint8_t* U = dst + t.pool_off;
  if ((dv % 16) == 0 && (t.pool_off % 16) == 0) {
    const int per = dv / 16;
    for (int q = tid; q < r * per; q += kThreads) {
      const int j = q / per, o = q % per;
      st_stream(*reinterpret_cast<const u32x4*>(&qbuf[j * kQStride + 16 * o]),
                reinterpret_cast<u32x4*>(U + j * dv + 16 * o));
    }
  } else {
    const int per = dv / 4;
    for (int q = tid; q < r * per; q += kThreads) {
      const int j = q / per, o = q % per;
      *reinterpret_cast<uint32_t*>(U + j * dv + 4 * o) =
          *reinterpret_cast<const uint32_t*>(&qbuf[j * kQStride + 4 * o]);
    }
  }
}

// INT8 pack of 32-column blocks of d = 128 heads (all 128 rows, 16 KiB a
// block): lane (v8, cg), v8 = tid / 8, cg = tid % 8, holds rows 4 v8 ..
// 4 v8 + 3 of channels 32 cb + 4 cg .. + 3 (one 16-byte load per row; 8
// lanes cover a 128-byte row segment).  The column maxima are combined over
// the 8 row lanes of a wave by lane exchanges and over the 4 waves in LDS.
//
// The loads are buffer loads over the head's 64 KiB; a block that is not
// packed (a KDA block without a retained channel) is given range 0, whose
// loads return zeros without touching memory, so that every block issues
// the same loads and the waits before a block's first use stay partial.
__device__ __forceinline__ void qblock_load(const uint8_t* head, bool live, int cb, f32x4 (&x)[4]) {
  const int tid = threadIdx.x, v8 = tid >> 3, cg = tid & 7;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(head), 0, live ? 128 * 128 * 4 : 0, 0x00020000);
  const int off = 128 * cb + 16 * cg + 4 * v8 * 512;  // row 4 v8, channel 32 cb + 4 cg
#pragma unroll
  for (int i = 0; i < 4; ++i)
    x[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 512 * i, 0, 2));  // slc
}

// Scales of the lane's four columns: s = max(a, 1e-8) / 127 and 1 / s.
__device__ __forceinline__ void qblock_scales(const f32x4 (&x)[4], float (&red)[8][128], f32x4& sc,
                                              f32x4& inv) {
  const int tid = threadIdx.x, cg = tid & 7, wave = tid >> 6;
  f32x4 mx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float m = fabsf(x[i][c]);
      mx[c] = m > mx[c] ? m : mx[c];  // NaN entries never win
    }
#pragma unroll
  for (int sh = 8; sh < 64; sh <<= 1) {  // the wave's 8 row lanes of this cg
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float o = __shfl_xor(mx[c], sh);
      mx[c] = o > mx[c] ? o : mx[c];
    }
  }
  if ((tid & 63) < 8) *reinterpret_cast<f32x4*>(&red[wave][4 * cg]) = mx;
  __syncthreads();
  // One lane per column (lanes 0 .. 31 of wave 0) combines the 4 waves'
  // maxima and divides once; every lane reads its columns' scale and
  // reciprocal back (the divisions are most of the block's arithmetic
  // when every lane repeats them).
  if (tid < 32) {
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) m = red[w][tid] > m ? red[w][tid] : m;
    const float s = (m > kScaleFloor ? m : kScaleFloor) / 127.f;  // correctly rounded fp32 division
    red[4][tid] = s;
    red[5][tid] = 1.f / s;
  }
  __syncthreads();
  sc = *reinterpret_cast<const f32x4*>(&red[4][4 * cg]);
  inv = *reinterpret_cast<const f32x4*>(&red[5][4 * cg]);
}

// A KDA head's block: each retained column's 4 bytes of the lane's rows go
// to its unit row in LDS (qbuf) and its scale to qs.  Segment j of the block
// is unit (retained channels below 32 cb) + j of the head.
__device__ __forceinline__ void qpack_kda_block(const Piece& t, int cb, const f32x4 (&x)[4],
                                                float (&red)[8][128], uint8_t* qbuf, float* qs) {
  const int tid = threadIdx.x, v8 = tid >> 3, cg = tid & 7;
  uint32_t bits4 = 0, below = 0;
  lane_ranks(t, 8 * cb + cg, bits4, below);
  f32x4 sc, inv;
  qblock_scales(x, red, sc, inv);
  uint32_t w[4];
  quant16(x, sc, inv, w);
  uint32_t b[4];
  transpose4(w, b);  // b[c]: column c, rows 4 v8 .. 4 v8 + 3
  uint32_t rk = below;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if ((bits4 >> c) & 1u) {
      *reinterpret_cast<uint32_t*>(&qbuf[rk * kQStride + 4 * v8]) = b[c];
      if (v8 == 0) qs[rk] = sc[c];
      ++rk;
    }
  }
}

// A GDN head's block: the codes of the lane's 4 rows x 4 columns go to the
// head's int8 rows in LDS (qbuf, row v at v kQStride), the scales of its
// columns to qs.
__device__ __forceinline__ void qpack_gdn_block(int cb, const f32x4 (&x)[4], float (&red)[8][128],
                                                uint8_t* qbuf, float* qs) {
  const int tid = threadIdx.x, v8 = tid >> 3, cg = tid & 7;
  f32x4 sc, inv;
  qblock_scales(x, red, sc, inv);
  uint32_t w[4];
  quant16(x, sc, inv, w);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint32_t*>(&qbuf[(4 * v8 + i) * kQStride + 32 * cb + 4 * cg]) = w[i];
  if (v8 == 0) *reinterpret_cast<f32x4*>(&qs[32 * cb + 4 * cg]) = sc;
}

// A d = 128 head's four 32-column blocks: the loads of all four (the head's
// 64 KiB) are issued first, then the blocks are reduced, scaled and
// quantized one after the other (a barrier waits only for LDS traffic, so
// the later blocks' loads stay in flight across the earlier blocks'
// barriers).  The codes and scales collect in LDS and leave after the last
// block as whole 128-byte lines: a store issued between the loads would
// hold the next block's first use until the store completes (one counter
// tracks loads and stores, in order), and one workgroup writing all of a
// head's int8 rows needs no partial-line writes.  Measured INT8 pack rates
// (GDN / mixed / KDA workloads, one box): 0.71 / 0.72 / 0.71 of the HBM peak
// with all four blocks in flight (100 VGPRs, 4 workgroups a CU), 0.71 /
// 0.70 / 0.67 with two blocks ahead of the one in hand, 0.70 / 0.67 / 0.66
// with one, 0.63 / 0.65 / 0.67 as one block a workgroup (a head's blocks
// placed on one XCD, stores after each block).  A KDA block without a
// retained channel loads nothing and is skipped (uniform per workgroup).
__device__ __forceinline__ void qpack_head_blocks(const Piece& t, const uint8_t* src, uint8_t* dst,
                                                  float (&red)[8][128], uint8_t* qbuf, float* qs) {
  constexpr int D = 128;
  const int tid = threadIdx.x;
  const bool gdn = t.type == kPieceQGdnBlock;
  const uint8_t* head = src + t.dense_off;
  f32x4 x[4][4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) qblock_load(head, gdn || mask_word(t, cb) != 0, cb, x[cb]);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    if (gdn) qpack_gdn_block(cb, x[cb], red, qbuf, qs);
    else if (mask_word(t, cb) != 0) qpack_kda_block(t, cb, x[cb], red, qbuf, qs);
  }
  __syncthreads();
  // GDN: the head's d_v int8 rows; KDA: its r units.  Both are rows of 128
  // bytes, 8 lanes to a row in 16-byte pieces, or 32 lanes in 4-byte words
  // where the payload offset is not 16-byte aligned (a layer before this one
  // with d_v not a multiple of 16 leaves the INT8 payload 4-byte aligned).
  const int rows = gdn ? D : t.r;
  uint8_t* U = dst + t.pool_off;
  if ((t.pool_off & 15u) == 0) {  // uniform
#pragma unroll
    for (int k = 0; k < D * 8 / kThreads; ++k) {
      const int q = tid + k * kThreads, row = q >> 3, g = q & 7;
      if (row < rows)
        st_stream(*reinterpret_cast<const u32x4*>(&qbuf[row * kQStride + 16 * g]),
                  reinterpret_cast<u32x4*>(U + row * D + 16 * g));
    }
  } else {
#pragma unroll
    for (int k = 0; k < D * 32 / kThreads; ++k) {
      const int q = tid + k * kThreads, row = q >> 5, w = q & 31;
      if (row < rows)
        *reinterpret_cast<uint32_t*>(U + row * D + 4 * w) =
            *reinterpret_cast<const uint32_t*>(&qbuf[row * kQStride + 4 * w]);
    }
  }
  if (tid < rows) reinterpret_cast<float*>(dst + t.scale_off)[tid] = qs[tid];  // GDN: 128 columns
}

// Unpack of kQGdnRows rows of a GDN head: lane (vl, kg) writes columns
// 4 kg .. 4 kg + 3 of rows kQGdnRows rb + 8 i + vl (every store instruction
// of the workgroup covers 8 consecutive rows); the int8 words are all loaded
// before the first store.
__device__ __forceinline__ void qunpack_gdn_rows(const Piece& t, const uint8_t* src, uint8_t* dst) {
  constexpr int kPer = kQGdnRows / 8;  // rows per lane
  const int dk = t.d_k, dv = t.d_v, KG = dk / 4;
  const int tid = threadIdx.x, kg = tid % 32, vl = tid / 32;
  if (kg >= KG) return;
  float* S = reinterpret_cast<float*>(dst + t.dense_off);
  const uint8_t* Sc = src + t.scale_off;
  const f32x4 sc = {load_scale(Sc + 16 * kg), load_scale(Sc + 16 * kg + 4),
                    load_scale(Sc + 16 * kg + 8), load_scale(Sc + 16 * kg + 12)};
  uint32_t w[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = kQGdnRows * t.rb + 8 * i + vl;
    w[i] = v < dv ? *reinterpret_cast<const uint32_t*>(src + t.pool_off + v * dk + 4 * kg) : 0u;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = kQGdnRows * t.rb + 8 * i + vl;
    if (v < dv) st_stream(dequant4(w[i], sc), reinterpret_cast<f32x4*>(S + v * dk + 4 * kg));
  }
}

// Unpack of a KDA head, whole: units and scales into LDS, then every element.
__device__ __forceinline__ void qunpack_kda_head(const Piece& t, const uint8_t* src, uint8_t* dst,
                                                 uint8_t* qbuf, float* qs) {
  const int dk = t.d_k, dv = t.d_v, KG = dk / 4;
  const int tid = threadIdx.x, kg = tid % 32, vl = tid / 32;
  uint32_t bits4 = 0, below = 0;
  lane_ranks(t, kg, bits4, below);
  float* S = reinterpret_cast<float*>(dst + t.dense_off);
  const int r = t.r;
  const uint8_t* U = src + t.pool_off;
  if ((dv % 16) == 0 && (t.pool_off % 16) == 0) {
    const int per = dv / 16;
    for (int q = tid; q < r * per; q += kThreads) {  // plain loads: measured faster here
      const int j = q / per, o = q % per;
      *reinterpret_cast<u32x4*>(&qbuf[j * kQStride + 16 * o]) =
          *reinterpret_cast<const u32x4*>(U + j * dv + 16 * o);
    }
  } else {
    const int per = dv / 4;
    for (int q = tid; q < r * per; q += kThreads) {
      const int j = q / per, o = q % per;
      *reinterpret_cast<uint32_t*>(&qbuf[j * kQStride + 4 * o]) =
          *reinterpret_cast<const uint32_t*>(U + j * dv + 4 * o);
    }
  }
  if (tid < r) qs[tid] = load_scale(src + t.scale_off + 4 * tid);
  __syncthreads();
  if (kg >= KG) return;
  // the 16 bytes of rows 16 vl .. 16 vl + 15 of each of this lane's columns;
  // an omitted column reads as q = 0 with scale 0, i.e. +0.0
  uint32_t cw[4][4];  // [column c][row group m]
  f32x4 s;
  uint32_t rk = below;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4 q = {0u, 0u, 0u, 0u};
    s[c] = 0.f;
    if ((bits4 >> c) & 1u) {
      q = *reinterpret_cast<const u32x4*>(&qbuf[rk * kQStride + 16 * vl]);
      s[c] = qs[rk];
      ++rk;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) cw[c][m] = q[m];
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t w[4] = {cw[0][m], cw[1][m], cw[2][m], cw[3][m]};
    uint32_t rows[4];
    transpose4(w, rows);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = kQRows * vl + 4 * m + i;
      if (v < dv)
        st_stream(dequant4(rows[i], s), reinterpret_cast<f32x4*>(S + v * dk + 4 * kg));
    }
  }
}

// kBlocks (pack lists of copy pieces and KDA column blocks only): an
// instantiation without the whole-head code, whose 64 VGPRs of rows would
// otherwise hold every workgroup of the launch to four per CU.
template <bool kPack, bool kBlocks = false>
__global__ void __launch_bounds__(kThreads) qmove_kernel(MoveArgs a) {
  static_assert(kPack || !kBlocks, "block lists are pack lists");
  __shared__ __attribute__((aligned(16))) float red[kPack ? 8 : 1][128];  // column maxima per row lane
  __shared__ __attribute__((aligned(16))) uint8_t qbuf[128 * kQStride];  // int8 rows / units
  __shared__ __attribute__((aligned(16))) float qs[128];                 // scales
  const Piece t = load_piece(a.pieces, blockIdx.x);
  const int64_t si = a.src_idx[blockIdx.y];
  const int64_t di = a.dst_idx[blockIdx.y];
  const bool bad_idx = !in_range(si, a.n_src) || !in_range(di, a.n_dst);
  const bool block = kPack && (t.type == kPieceQKdaBlock || t.type == kPieceQGdnBlock);
  const bool valid = kBlocks ? (t.type == kPieceCopy || block) : (t.type <= kPieceQKda || block);
  if (bad_idx | !valid) {
    if (bad_idx && blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, DASC_STATUS_BAD_INDEX);
    return;
  }
  const uint8_t* src = a.src_base + si * a.src_stride;
  uint8_t* dst = a.dst_base + di * a.dst_stride;
  if (t.type == kPieceCopy || t.type == kPieceZero) {
    copy_piece<kPack>(t, src, dst);
    return;
  }
  if constexpr (kBlocks) {
    qpack_head_blocks(t, src, dst, red, qbuf, qs);
  } else if constexpr (kPack) {
    if (t.type == kPieceQGdnBlock || t.type == kPieceQKdaBlock)
      qpack_head_blocks(t, src, dst, red, qbuf, qs);
    else if (t.type == kPieceQKda)
      qpack_kda_head(t, src, dst, red, qbuf);
    else
      qpack_gdn_head(t, src, dst, red);
  } else {
    if (t.type == kPieceQKda)
      qunpack_kda_head(t, src, dst, qbuf, qs);
    else
      qunpack_gdn_rows(t, src, dst);
  }
}

// ---------------------------------------------------------------------------
// Bounded-suffix refresh ([dasc] §4.2), one workgroup per (head, request).
//
// Eq. 1 ([dasc] §3.1) is replayed in chunks of 16 tokens.  Inside a chunk
// that starts from S_0, with the running decay gamma_t = alpha_0 ... alpha_t
// and the pairwise decay D_{t,s} = alpha_{s+1} ... alpha_t (s < t), the
// recurrence unrolls exactly to
//   S_t = S_0 Diag(gamma_t) + sum_{s<=t} c_s (k_s o D_{t,s})^T,
//   (I + L) c = R,  R_t = beta_t (v_t - S_0 (gamma_t o k_t)),
//   L_{t,s} = beta_t sum_j k_t[j] k_s[j] D_{t,s}[j]   (s < t),
// so a chunk is one product U0 = S_0 Q (Q = [gamma_t o k_t]), C = T R with
// the 16 x 16 unit-lower-triangular inverse T = (I + L)^-1, and one rank-16
// update S_16 = S_0 Diag(gamma_15) + sum_s c_s w_s^T (w_s = k_s o D_{15,s}).
// Every factor is a product of decays, so nothing is divided (channels
// whose decay underflows cannot overflow anything).  Tokens past the end of
// a request pad the last chunk as exact no-ops (alpha = 1, k = v = 0,
// beta = 0).
//
// The three products run on MFMA.  For d <= 32 all three are fp32
// (v_mfma_f32_16x16x4f32); for d >= 64 the readout and the update use bf16
// hi / lo splits of both operands (v_mfma_f32_16x16x32_bf16, hi hi + hi lo +
// lo hi with fp32 accumulation: fp32 MFMA runs at the fp32 vector rate on
// gfx950 and does not overlap the VALU work, bf16 moves 8x the MACs per
// instruction), and C = T R stays fp32.  The state is kept transposed,
// S^T [k][v], in 16 x 16 accumulator tiles: lane (g, m)
// (g = lane / 16, m = lane % 16) of tile (kt, vt) holds
// S^T[16 kt + 4 g + r][16 vt + m], r = 0..3.  With the K index of k-step r
// read as 4 g + r on both operands, those same registers are the B operand
// of the readout, and every product's output is the next one's B operand:
//   U0^T[t][v] = sum_k Q[t][k] S^T[k][v]   (A = Q from LDS, B = S^T)
//   C[t][v]    = sum_s T[t][s] R[s][v]     (A = T from LDS, B = R)
//   S^T[k][v] += sum_t W[k][t] C[t][v]     (A = W from LDS, B = C)
// (with bf16 operands two k tiles, or the C hi and lo halves, fill the 8 K
// slots of a lane group), so the state never moves.  Each wave owns all k tiles of its v tiles: no
// product needs a cross-wave reduction.
//
// Software pipeline.  The chunk inputs (decays from the gate logits by
// Eq. 2 ([dasc] §3.3), Q, W, gamma_15, L, T) do not depend on the state, so
// chunk n + 1 is prepared while chunk n runs its products:
//   phase 1: T(n) = (I + L(n))^-1; U0 = S Q(n)  ||  stage chunk n + 1
//            (decays, k, v, beta into LDS); fetch chunk n + 2
//   phase 2: R, C = T R; S <- S Diag(gamma) + W C  ||  L(n + 1), gamma,
//            Q(n + 1), W(n + 1)
// with one barrier after each phase; T(n) is computed by one wave per chunk,
// rotating.  The two workgroups a CU holds overlap each other's phases.
// LDS buffers that live across an iteration are double-buffered by chunk
// parity; staging and fetches past the request's last chunk are skipped.
// ---------------------------------------------------------------------------
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kC = kRefreshChunk;

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <int D>
struct RefreshShape {
  static constexpr int kKT = D / 16;                  // k tiles
  static constexpr bool kSplit = D >= 64;             // big products on split bf16 MFMA
  static constexpr int kWavesPerSimd = 2;  // occupancy target
  static constexpr int kWavesPerSimdOne = 4;  // ... of the one-chunk kernel
  // ... of the one-chunk kernel over KDA heads of d = 128, which reads the
  // old rows of its whole-row write-back before the replay
  static constexpr int kWavesPerSimdOneEarly = D == 128 ? 2 : 4;
  static constexpr int kVTW = D >= 32 ? 2 : 1;        // v tiles per wave
  static constexpr int kNW = (D / 16) / kVTW;         // waves per head
  static constexpr int kNT = 64 * kNW;                // threads
  static constexpr int kJB = D / 8;                   // 8-channel blocks per token
  static constexpr int kNB4 = D / 4;                  // lanes per row pair of L
  static_assert(2 * D <= kNT, "one staged item per lane");
};

// Q and W in fp32 (d <= 32) or as bf16 hi / lo pairs (the split products).
// NB: buffers by chunk parity (2; 1 for the one-chunk kernel, which has no
// Q: its readout meets the zero state only).
template <int D, bool SPLIT, int NB>
struct RefreshQW {
  float Q[NB == 2 ? kC : 1][D + 4];  // gamma_t o k_t
  float W[NB][D][kC + 4];            // k_s o D_{15,s}, [k][s], by chunk parity
};
template <int D, int NB>
struct RefreshQW<D, true, NB> {
  // gamma_t o k_t: bf16 hi, then lo.  Rows padded by 16 bytes: the 16 rows
  // m of one 8-byte A-operand read start 4 banks apart.
  uint16_t Qh[NB == 2 ? kC : 1][D + 8];
  uint16_t Ql[NB == 2 ? kC : 1][D + 8];
  // k_s o D_{15,s}, [k][s], by chunk parity: per row k and token group
  // g (s = 4 g .. 4 g + 3) the four bf16 hi, then the four bf16 lo.  Rows
  // are padded to 80 bytes (20 banks), so the 16 rows that one 16-byte
  // A-operand read spans start on 16 different 4-bank groups.
  uint16_t W[NB][D][2 * kC + 8];
};

template <int D, int NB>
struct alignas(16) RefreshLds {
  float K[kC][D];             // k of the chunk being prepared
  float A[kC][D];             // its decays
  // v (bf16 bits as given), by chunk parity; rows padded by 16 bytes, so
  // the rows 4 g + r that the lane groups g read at once fall on
  // disjoint banks
  uint16_t V[NB][kC][D + 8];
  float B[NB][kC];            // beta, by chunk parity
  RefreshQW<D, RefreshShape<D>::kSplit, NB> qw;
  float G[NB][D];             // gamma_15 by chunk parity
  float PA[D], PD[D];         // exp(A_log) and dt_bias per channel (GDN: [0])
  float LT[kC][kC + 4];       // L transposed: LT[s][t] = beta_t M_{t,s}, s < t
  float T[kC][kC + 4];        // (I + L)^-1
  float Xt[8][8 + 4];         // the inverse's L21 T11, transposed
};

// Split of an fp32 value into bf16 hi + lo (hi = x truncated to bf16, lo =
// the remainder x - hi, exact in fp32, truncated to bf16): x = hi + lo to a
// relative 2^-16.  A product of two split values is taken as
// hi hi + hi lo + lo hi on bf16 MFMA with fp32 accumulation; the dropped
// lo lo term and the truncations are below 2^-15 of each product term.
// The remainder is never fused with a product that computes x (fp
// contraction would split the exact product instead of the rounded x, and
// kernels that inline the split into different code would then disagree).
__device__ __forceinline__ uint32_t hi_bits(float x) { return __float_as_uint(x) & 0xFFFF0000u; }
__device__ __forceinline__ uint32_t lo_bits(float x) {
#pragma clang fp contract(off)
  return __float_as_uint(x - __uint_as_float(hi_bits(x)));
}
// Two bf16 (the upper halves of a and b) in one word: a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4f mfma_bf16(u32x4 a, u32x4 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                 __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// alpha = exp(-exp(A_log) softplus(x)) with x = a_t + dt_bias (Eq. 2);
// expA = exp(A_log) is precomputed per unit.  softplus(x) = max(x, 0) +
// log(1 + z) with z = exp(-|x|) in (0, 1]; u = 1 + z is rounded, and the
// term z - (u - 1) restores what the rounding lost (its 1/u factor is at
// most a factor 2 away from 1 and the term itself is below 2^-24, so the
// factor is dropped), so log(1 + z) keeps full relative precision for small
// z.  Hardware exp2 / log2, a few ulp overall.
__device__ __forceinline__ float decay(float x, float expA) {
  constexpr float kLog2e = 1.44269504088896341f, kLn2 = 0.693147180559945309f;
  const float z = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float u = 1.f + z;
  const float l1p = __builtin_amdgcn_logf(u) * kLn2 + (z - (u - 1.f));
  const float sp = fmaxf(x, 0.f) + l1p;
  return __builtin_amdgcn_exp2f(-expA * sp * kLog2e);
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

// Sum over the G consecutive lanes of a 16-lane row (G in {1, 2, 4, 8, 16});
// every lane of the group gets the sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (G >= 16) x += dpp<0x140>(x); // row_mirror
  return x;
}

// One step of a reduce-scatter over the 16 lanes of a row: the lane and its
// DPP partner (kCtrl) hold the same 2N entries in v[0 .. 2N); the lane keeps
// the half its `upper` flag names, sends the other half, and adds what the
// partner sends, so that v[0 .. N) holds its half summed over both lanes.
template <int N, int kCtrl>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[16], bool upper) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float keep = upper ? v[i + N] : v[i];
    const float send = upper ? v[i] : v[i + N];
    v[i] = keep + dpp<kCtrl>(send);
  }
}

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// WINDOWED: each task replays only the last `window` tokens of its request
// (a kernel of its own, so that profiles tell the two refreshes apart).
// FUSED: the load and the refresh in one pass: the head is written whole,
// the local columns from the replay and the retained ones from its units in
// the pool slot (what a zero-fill unpack followed by the refresh leaves).
// ONE (with WINDOWED, chosen when every window of the launch is at most one
// chunk, so that every head replays at most kC tokens): the pipeline's
// staging of later chunks and the parity buffers are left out, which frees
// LDS and registers for four workgroups per CU (two for KDA heads of d =
// 128, whose registers go to reading the write-back's old rows early);
// short replays are bound by each head's serial chain (stage, L, T,
// products, write-back), which more resident heads overlap.
template <int D, int GATE, bool WINDOWED, bool FUSED, bool ONE>
__global__ void __launch_bounds__(RefreshShape<D>::kNT)
    __attribute__((amdgpu_waves_per_eu(ONE ? (GATE != kGateHead && GATE != kGateAlphaHead && !FUSED
                                                  ? RefreshShape<D>::kWavesPerSimdOneEarly
                                                  : RefreshShape<D>::kWavesPerSimdOne)
                                           : RefreshShape<D>::kWavesPerSimd)))
refresh_kernel(RefreshArgs a) {
  static_assert(!ONE || WINDOWED, "the one-chunk kernel serves windowed replays");
  using Sh = RefreshShape<D>;
  constexpr int KT = Sh::kKT, VTW = Sh::kVTW, JB = Sh::kJB, NB4 = Sh::kNB4;
  constexpr bool kAlpha = GATE >= kGateAlphaHead;  // decays given as fp32
  constexpr bool kChan = GATE != kGateHead && GATE != kGateAlphaHead;
  constexpr bool kGram = !kChan && Sh::kSplit;  // GDN heads, d >= 64: L from the Gram matrix
  constexpr bool kAllStage = Sh::kNT == 2 * D;  // every lane stages an item
  __shared__ RefreshLds<D, ONE ? 1 : 2> sh;

  const RefreshTask task = a.tasks[blockIdx.x];
  const int req = blockIdx.y;
  int64_t t0 = a.tok_off[req];
  const int64_t t1 = a.tok_off[req + 1];
  const int64_t dst = a.dst_idx[req];
  if (t0 < 0 || t1 < t0 || t1 > a.n_tokens) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, DASC_STATUS_BAD_TOKENS);
    return;
  }
  // Per-head Eq. 7 window: replay only the request's last `window` tokens.
  if constexpr (WINDOWED) t0 = t1 - t0 > task.window ? t1 - task.window : t0;
  if (!in_range(dst, a.n_dense)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, DASC_STATUS_BAD_INDEX);
    return;
  }
  const int64_t slot = FUSED ? a.src_slot[req] : 0;
  if (FUSED && !in_range(slot, a.n_slots)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, DASC_STATUS_BAD_INDEX);
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;  // wave w owns v tiles w VTW ..
  const int g = lane >> 4, m = lane & 15;

  // Staged item of this lane: token it_t of a chunk, channels j0 .. j0 + 7.
  const bool it_on = kAllStage || tid < 2 * D;
  const int it_t = (tid / JB) % kC, it_jb = tid % JB, j0 = 8 * it_jb;

  // Inputs of one token for this lane (8 bf16 of k, v and the gate logits,
  // packed, or 8 fp32 decays in ra and ra2, and beta), fetched one chunk
  // ahead of their staging.  The row is clamped into the request, so every
  // load is in bounds; past the end the values are replaced by the no-op
  // token when staged.  Token indices are below 2^31 (the host checks
  // n_tokens) and row widths below 2^32, so a row's offset is one 32 x 32
  // -> 64-bit multiply-add.
  const uint32_t t0u = static_cast<uint32_t>(t0), t1u = static_cast<uint32_t>(t1);
  const uint32_t k_row = static_cast<uint32_t>(a.k_row), v_row = static_cast<uint32_t>(a.v_row);
  const uint32_t g_row = static_cast<uint32_t>(a.g_row), b_row = static_cast<uint32_t>(a.b_row);
  u32x4 rk, rv, ra, ra2;
  float rb;
  bool r_real;
  auto fetch = [&](int64_t n) {
    const uint32_t tok = t0u + static_cast<uint32_t>(n) * kC + it_t;
    r_real = tok < t1u;
    const uint64_t tc = r_real ? tok : t1u - 1;
    rk = *reinterpret_cast<const u32x4*>(a.k + tc * k_row + task.k_off + j0);
    rv = *reinterpret_cast<const u32x4*>(a.v + tc * v_row + task.v_off + j0);
    if constexpr (kAlpha) {
      const float* pp = a.alpha + tc * g_row + task.g_off;
      if constexpr (GATE == kGateAlphaChan) {
        ra = *reinterpret_cast<const u32x4*>(pp + j0);
        ra2 = *reinterpret_cast<const u32x4*>(pp + j0 + 4);
      } else if constexpr (GATE == kGateAlphaChanSplit) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ra[q] = __float_as_uint(pp[j0 + q]);
          ra2[q] = __float_as_uint(pp[j0 + 4 + q]);
        }
      } else {
        ra = u32x4{__float_as_uint(pp[0]), 0u, 0u, 0u};
      }
    } else {
      const uint16_t* ap = a.a + tc * g_row + task.g_off;
      if constexpr (GATE == kGateChan) {
        ra = *reinterpret_cast<const u32x4*>(ap + j0);
      } else if constexpr (GATE == kGateChanSplit) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ra[q] = static_cast<uint32_t>(ap[j0 + 2 * q]) |
                  (static_cast<uint32_t>(ap[j0 + 2 * q + 1]) << 16);
      } else {
        ra = u32x4{static_cast<uint32_t>(ap[0]), 0u, 0u, 0u};
      }
    }
    rb = a.beta[tc * b_row + task.b_off];
  };

  // Stage the fetched token into LDS buffer vb: decays (given, or by Eq. 2),
  // k, v, beta.  A token past the end becomes a no-op: beta = 0 and a decay
  // of exactly 1 (given decays are replaced by 1; for logits a zero gate
  // scale makes the decay exp2(-0) = 1).  Its k and v (the last token's,
  // finite) then meet only zero factors: its row of L is beta k = 0, so its
  // row of T is the unit row and its entry of C = T R is R_t = beta (v -
  // u) = 0, and no earlier token's entry reads it (T is lower triangular).
  // (The padding is applied to inputs, not by selecting results, so the
  // code has no branch.)
  auto stage1 = [&](int vb) {
    float kf[8], al[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      kf[2 * q] = bf16_lo(rk[q]);
      kf[2 * q + 1] = bf16_hi(rk[q]);
    }
    if constexpr (kAlpha && kChan) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        al[q] = r_real ? __uint_as_float(ra[q]) : 1.f;
        al[q + 4] = r_real ? __uint_as_float(ra2[q]) : 1.f;
      }
    } else if constexpr (kAlpha) {
      const float x = r_real ? __uint_as_float(ra[0]) : 1.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) al[c] = x;
    } else if constexpr (kChan) {
      const v4f e0 = *reinterpret_cast<const v4f*>(&sh.PA[j0]);
      const v4f e1 = *reinterpret_cast<const v4f*>(&sh.PA[j0 + 4]);
      const v4f d0 = *reinterpret_cast<const v4f*>(&sh.PD[j0]);
      const v4f d1 = *reinterpret_cast<const v4f*>(&sh.PD[j0 + 4]);
      const float expA[8] = {e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]};
      const float dtb[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        al[2 * q] = decay(bf16_lo(ra[q]) + dtb[2 * q], r_real ? expA[2 * q] : 0.f);
        al[2 * q + 1] = decay(bf16_hi(ra[q]) + dtb[2 * q + 1], r_real ? expA[2 * q + 1] : 0.f);
      }
    } else {
      const float x = decay(bf16_lo(ra[0]) + sh.PD[0], r_real ? sh.PA[0] : 0.f);
#pragma unroll
      for (int c = 0; c < 8; ++c) al[c] = x;
    }
    const float bv = r_real ? rb : 0.f;
    if (it_on) {
      *reinterpret_cast<v4f*>(&sh.A[it_t][j0]) = v4f{al[0], al[1], al[2], al[3]};
      *reinterpret_cast<v4f*>(&sh.A[it_t][j0 + 4]) = v4f{al[4], al[5], al[6], al[7]};
      *reinterpret_cast<v4f*>(&sh.K[it_t][j0]) = v4f{kf[0], kf[1], kf[2], kf[3]};
      *reinterpret_cast<v4f*>(&sh.K[it_t][j0 + 4]) = v4f{kf[4], kf[5], kf[6], kf[7]};
      *reinterpret_cast<u32x4*>(&sh.V[vb][it_t][j0]) = rv;
      sh.B[vb][it_t] = bv;  // the JB lanes of a token store the same value
    }
  };

  // From the staged chunk: L (into sh.L), Q (sh.Q), W and gamma_15 (buffer vb).
  // PW >= 0 (d = 128, four waves): the caller's wave index, a compile-time
  // constant, so that the row pair of each half-wave (p = 2 PW + h) and the
  // direction of the Q / W lanes are known to the compiler and the only
  // per-lane selects left are at the two entries where the half-waves'
  // rows differ; PW = -1: the same work with p and the direction per lane.
  // L of a chunk of a GDN head (d >= 64), on wave 0: with one decay per
  // head and token, L_{t,s} = beta_t D_{t,s} (k_t . k_s) with the scalar
  // D_{t,s} = alpha_{s+1} ... alpha_t, and the keys are bf16 values, so the
  // Gram matrix G = K K^T comes exact in its products from bf16 MFMA (fp32
  // sums; one operand serves as A and B).  Lane (g, m) gets G[4 g + r][m]
  // and makes L[t][s] for t = 4 g + r, s = m: the running product of the
  // decays after s is captured at each of its rows t; entries with t <= s
  // are stored as zeros (the inverse never reads them).
  auto gram_L = [&](int vb) __attribute__((always_inline)) {
    if (wave != 0) return;  // uniform
    v4f G = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const v4f a0 = *reinterpret_cast<const v4f*>(&sh.K[m][32 * kk + 8 * g]);
      const v4f a1 = *reinterpret_cast<const v4f*>(&sh.K[m][32 * kk + 8 * g + 4]);
      const u32x4 ka = {pack_bf16(__float_as_uint(a0[0]), __float_as_uint(a0[1])),
                        pack_bf16(__float_as_uint(a0[2]), __float_as_uint(a0[3])),
                        pack_bf16(__float_as_uint(a1[0]), __float_as_uint(a1[1])),
                        pack_bf16(__float_as_uint(a1[2]), __float_as_uint(a1[3]))};
      G = mfma_bf16(ka, ka, G);
    }
    float run = 1.f;
    v4f dr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 1; u < kC; ++u) {
      run *= u > m ? sh.A[u][0] : 1.f;  // D_{u,m} once u > m
      if ((u >> 2) == g) dr[u & 3] = run;
    }
    const v4f b4 = *reinterpret_cast<const v4f*>(&sh.B[vb][4 * g]);
    v4f l4;
#pragma unroll
    for (int r = 0; r < 4; ++r) l4[r] = 4 * g + r > m ? b4[r] * dr[r] * G[r] : 0.f;
    *reinterpret_cast<v4f*>(&sh.LT[m][4 * g]) = l4;
  };

  auto stage2_body = [&](int vb, auto pw_c) __attribute__((always_inline)) {
    constexpr int PW = decltype(pw_c)::value;
    static_assert(PW < 0 || (NB4 == 32 && kAllStage), "wave-uniform rows need d = 128");
    if constexpr (kGram) gram_L(vb);
    if (kAllStage || tid < 2 * D) {
     if constexpr (!kGram) {
      // L, rows p and 15 - p (15 entries in all), 4 channels per lane,
      // summed over the NB4 lanes of the row pair after the loop (so the
      // loop has no branch): for NB4 = 32 by a reduce-scatter that leaves
      // one entry per lane, otherwise by DPP sums within a row whose last
      // lane stores every entry.
      // PW >= 0: lanes with bit 3 clear serve row pair 2 PW, the others
      // 2 PW + 1, so that both pairs span all four 16-lane rows and the
      // sums over a pair's lanes can cross rows with lane swaps (below).
      // Channel block ci of a lane: bits 0-2 from the lane, bits 3-4 from
      // its row, flipped for the second pair so that the two pairs of a
      // 16-lane row read different LDS banks.
      const bool h = PW >= 0 && (lane & 8) != 0;
      const int ci = PW >= 0 ? (lane & 7) | (((lane >> 4) ^ (h ? 1 : 0)) << 3) : tid % NB4;
      const int p = PW >= 0 ? 2 * PW + (h ? 1 : 0) : tid / NB4, c4 = 4 * ci;
      // entry i is in row p (i < p), and row 15 - p starts at i = p
      auto in_row_p = [&](int i) {
        return PW >= 0 ? (i < 2 * PW || (i == 2 * PW && h)) : i < p;
      };
      auto starts_q = [&](int i) {
        return PW >= 0 ? ((i == 2 * PW && !h) || (i == 2 * PW + 1 && h)) : i == p;
      };
      // K and A are adjacent [kC][D] arrays: row r of A is row kC + r here.
      const float(*KA)[D] = reinterpret_cast<const float(*)[D]>(&sh.K[0][0]);
      const float bp = sh.B[vb][p], bq = sh.B[vb][kC - 1 - p];
      v4f kp = *reinterpret_cast<const v4f*>(&KA[p][c4]);
      v4f kq = *reinterpret_cast<const v4f*>(&KA[kC - 1 - p][c4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // beta_t folded into the row's key
        kp[e] *= bp;
        kq[e] *= bq;
      }
      // Entry i: row p, s = p - 1 - i (i < p), else row 15 - p, s = 14 - i;
      // both walk down from a base row, so the addresses are a base chosen
      // per entry plus a constant.
      const float* const rowP = &KA[p][c4];
      const float* const rowQ = &KA[kC - 1][c4];
      v4f pk = kp;
      float lv[kC - 1];
#pragma unroll
      for (int i = 0; i < kC - 1; ++i) {
        const bool first = in_row_p(i);
        const float* const r0 = first ? rowP : rowQ;  // K row s + 1
        if (i == 0) pk = first ? kp : kq;
        else pk = starts_q(i) ? kq : pk;
        const v4f al = *reinterpret_cast<const v4f*>(r0 + (kC - i) * D);   // A[s + 1]
        const v4f ks = *reinterpret_cast<const v4f*>(r0 - (i + 1) * D);    // K[s]
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[e] *= al[e];
          part = fmaf(pk[e], ks[e], part);
        }
        if constexpr (NB4 != 32) part = group_sum<(NB4 < 16 ? NB4 : 16)>(part);
        lv[i] = part;
      }
      // L[p][p - 1 - i] and L[15 - p][14 - i], stored transposed: two
      // bases, constant steps
      float* const lP = &sh.LT[0][0] + (p - 1) * (kC + 4) + p;
      float* const lQ = &sh.LT[0][0] + (kC - 2) * (kC + 4) + (kC - 1 - p);
      if constexpr (PW >= 0) {
        // The 15 entries' partial sums (4 channels each) are summed over the
        // row pair's 32 lanes by a reduce-scatter.  Across rows, a lane swap
        // between two registers (v_permlane32_swap / v_permlane16_swap: the
        // upper half of the first register trades places with the lower
        // half of the second) gives each lane its kept entry from both
        // partners with one add and no select: the lanes 32 apart, then 16
        // apart.  Within the 8 lanes of a pair in a row, two DPP exchanges
        // halve the rest, and one more adds the last partner's sum.  The
        // lane keeps entry e = 8 b5 + 4 b4 + 2 b2 + b1 (b = its lane bits);
        // lanes with b0 = 0 store it.
        float v[16];
#pragma unroll
        for (int i = 0; i < kC - 1; ++i) v[i] = lv[i];
        v[15] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                          __float_as_uint(v[i + 8]), false, false);
          v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]),
                                                          __float_as_uint(v[i + 4]), false, false);
          v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
        reduce_scatter_step<2, 0x141>(v, (lane & 4) != 0);  // row_half_mirror: l <-> 7 - l
        reduce_scatter_step<1, 0x4E>(v, (lane & 2) != 0);   // quad_perm [2,3,0,1]
        const float sum = v[0] + dpp<0xB1>(v[0]);           // quad_perm [1,0,3,2]
        const int e = ((lane >> 2) & 8) | ((lane >> 2) & 4) | ((lane >> 1) & 2) | ((lane >> 1) & 1);
        if ((lane & 1) == 0 && e < kC - 1) *((in_row_p(e) ? lP : lQ) - e * (kC + 4)) = sum;
      } else if constexpr (NB4 == 32) {
        // The same sums for a lane layout known only at run time: four DPP
        // exchanges within each 16-lane row leave lane r16 with entry r16's
        // row sum, and one lane exchange across the two rows completes it;
        // lanes 0 .. 14 of the lower row then store one entry each.
        const int r16 = lane & 15;
        float v[16];
#pragma unroll
        for (int i = 0; i < kC - 1; ++i) v[i] = lv[i];
        v[15] = 0.f;
        reduce_scatter_step<8, 0x140>(v, (r16 & 8) != 0);  // row_mirror: l <-> 15 - l
        reduce_scatter_step<4, 0x141>(v, (r16 & 4) != 0);  // row_half_mirror
        reduce_scatter_step<2, 0x4E>(v, (r16 & 2) != 0);   // quad_perm [2,3,0,1]
        reduce_scatter_step<1, 0xB1>(v, (r16 & 1) != 0);   // quad_perm [1,0,3,2]
        const float sum = v[0] + __shfl_xor(v[0], 16);
        if ((lane & 16) == 0 && r16 < kC - 1)
          *((in_row_p(r16) ? lP : lQ) - r16 * (kC + 4)) = sum;
      } else if (tid % NB4 == NB4 - 1) {
#pragma unroll
        for (int i = 0; i < kC - 1; ++i) *((in_row_p(i) ? lP : lQ) - i * (kC + 4)) = lv[i];
      }
     }
      // gamma_t and Q (forward lanes, tid < D) or W (backward lanes)
      const int j = tid % D;
      const bool fwd = PW >= 0 ? PW < 2 : tid < D;
      float gm = 1.f;
      if constexpr (Sh::kSplit) {
        float qw[kC];  // step i: token i (forward) or token 15 - i (backward)
#pragma unroll
        for (int i = 0; i < kC; ++i) {
          const int t = fwd ? i : kC - 1 - i;
          const float al = sh.A[t][j], kv = sh.K[t][j];
          const float before = gm * kv;  // backward: k_s o D_{15,s}
          gm *= al;
          qw[i] = fwd ? gm * kv : before;  // forward: gamma_t o k_t
        }
        if (fwd) {
          if constexpr (!ONE) {
#pragma unroll
            for (int t = 0; t < kC; ++t) {
              sh.qw.Qh[t][j] = static_cast<uint16_t>(hi_bits(qw[t]) >> 16);
              sh.qw.Ql[t][j] = static_cast<uint16_t>(lo_bits(qw[t]) >> 16);
            }
          }
        } else {
#pragma unroll
          for (int gq = 0; gq < kC / 4; ++gq) {  // tokens s = 4 gq .. 4 gq + 3
            const float w0 = qw[kC - 1 - 4 * gq], w1 = qw[kC - 2 - 4 * gq];
            const float w2 = qw[kC - 3 - 4 * gq], w3 = qw[kC - 4 - 4 * gq];
            *reinterpret_cast<u32x4*>(&sh.qw.W[vb][j][8 * gq]) =
                u32x4{pack_bf16(hi_bits(w0), hi_bits(w1)), pack_bf16(hi_bits(w2), hi_bits(w3)),
                      pack_bf16(lo_bits(w0), lo_bits(w1)), pack_bf16(lo_bits(w2), lo_bits(w3))};
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kC; ++i) {
          const int t = fwd ? i : kC - 1 - i;
          const float al = sh.A[t][j], kv = sh.K[t][j];
          const float before = gm * kv;  // backward: k_s o D_{15,s}
          gm *= al;
          const float after = gm * kv;   // forward: gamma_t o k_t
          if constexpr (ONE) {
            if (!fwd) sh.qw.W[vb][j][t] = before;
          } else {
            float* const at = fwd ? &sh.qw.Q[t][j] : &sh.qw.W[vb][j][t];
            *at = fwd ? after : before;
          }
        }
      }
      if (!ONE && fwd) sh.G[vb][j] = gm;  // the one-chunk kernel decays a zero state
    }
  };
  auto stage2 = [&](int vb) __attribute__((always_inline)) {
    stage2_body(vb, IntC<-1>{});
  };
  // In the chunk loop: one specialized copy per wave (a uniform branch on
  // the wave index).
  auto stage2_waves = [&](int vb) __attribute__((always_inline)) {
    if constexpr (NB4 == 32 && kAllStage && Sh::kNW == 4) {
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      if (wv == 0) stage2_body(vb, IntC<0>{});
      else if (wv == 1) stage2_body(vb, IntC<1>{});
      else if (wv == 2) stage2_body(vb, IntC<2>{});
      else stage2_body(vb, IntC<3>{});
    } else {
      stage2_body(vb, IntC<-1>{});
    }
  };

  // T = (I + L)^-1 in 8 x 8 blocks: with L = [[L11, 0], [L21, L22]] the
  // inverse is [[T11, 0], [T21, T22]] with T11 = (I + L11)^-1,
  // T22 = (I + L22)^-1 and T21 = -T22 L21 T11.  One wave per chunk computes
  // it (its four 16-lane rows do the same work; their stores write the same
  // values); the others read T after the barrier that ends the phase.
  //  1. Lane sc = lane % 16 < 8 computes column sc of T11, lanes 8 .. 15
  //     column sc of T22 (block offset o), T[u][s] = delta_{us} -
  //     sum_{v<u} L[u][v] T[v][s] right-looking: as soon as T[u][s] is
  //     known it is added into the running sums of the later rows, so the
  //     dependent chain is one multiply-add per row (8 rows, not 16).  For
  //     u < s the sums only meet zeros, so one formula serves every row.
  //     Row u + 1 of L^T is loaded while row u is applied (the compiler
  //     fence keeps it from hoisting every load).
  //  2. Every lane takes column lane % 8 of T11 (DPP within its row), and
  //     lane (t, s) = (8 + lane / 8, lane % 8) forms X = L21 T11 at (t, s),
  //     stored transposed, then T21[t][s] = -sum_u T22[t][u] X[u][s].
  // T12 stays zero (cleared once before the chunk loop).
  auto invert = [&]() {
    const int sc = lane & 15, o = sc & 8;
    float run[8], tc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) run[t] = 0.f;
    v4f rowv[2][2];
    rowv[0][0] = *reinterpret_cast<const v4f*>(&sh.LT[o][o]);
    rowv[0][1] = *reinterpret_cast<const v4f*>(&sh.LT[o][o + 4]);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u + 1 < 7) {
#pragma unroll
        for (int q = (u + 2) / 4; q < 2; ++q)
          rowv[(u + 1) & 1][q] = *reinterpret_cast<const v4f*>(&sh.LT[o + u + 1][o + 4 * q]);
      }
      const float tu = (o + u == sc ? 1.f : 0.f) - run[u];
      tc[u] = tu;
#pragma unroll
      for (int q = (u + 1) / 4; q < 2; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q + e > u) run[4 * q + e] = fmaf(rowv[u & 1][q][e], tu, run[4 * q + e]);
      }
      sh.T[o + u][sc] = tu;
      __asm__ volatile("" ::: "memory");
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)  // row_ror:8 into lanes 8 .. 15 of each row (banks 2, 3)
      tc[u] = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(tc[u]),
                                                         __float_as_int(tc[u]), 0x128, 0xF, 0xC, false));
    const int t = 8 + (lane >> 3), s = lane & 7;
    float x = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) x = fmaf(sh.LT[u][t], tc[u], x);  // L[t][u] = LT[u][t]
    sh.Xt[s][t - 8] = x;
    const v4f a0 = *reinterpret_cast<const v4f*>(&sh.T[t][8]);
    const v4f a1 = *reinterpret_cast<const v4f*>(&sh.T[t][12]);
    const v4f x0 = *reinterpret_cast<const v4f*>(&sh.Xt[s][0]);
    const v4f x1 = *reinterpret_cast<const v4f*>(&sh.Xt[s][4]);
    float y = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y = fmaf(a0[e], x0[e], y);
      y = fmaf(a1[e], x1[e], y);
    }
    sh.T[t][s] = -y;
  };

  // Write-back of the windowed refresh (below): heads that also hold
  // retained columns are written as whole rows merged with the rows' old
  // contents.  The one-chunk kernel reads those old rows here, before the
  // replay, so that the reads are in flight while it computes (1.12 -> 1.10
  // ms on the KDA windows, at two waves per SIMD instead of four).
  float* const out = reinterpret_cast<float*>(a.dense + dst * a.dense_stride + task.dense_off);
  constexpr int LPR = D / 4, RPI = 64 / LPR, NI = 16 / RPI;  // lanes a row, rows a store, stores a tile
  const int c4 = lane % LPR, rsub = lane / LPR;
  bool rmw = WINDOWED;  // (uniform) whole rows, unless every channel of the head is local
  if constexpr (WINDOWED) {
    bool all_local = true;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t want =
          32 * q >= D ? 0u : (D - 32 * q >= 32 ? 0xFFFFFFFFu : (1u << (D - 32 * q)) - 1u);
      all_local = all_local && (task.local[q] & want) == want;
    }
    rmw = !all_local;
  }
  constexpr bool kEarly = ONE && !FUSED && kChan;  // GDN heads are all local: no old rows
  v4f old[kEarly ? VTW : 1][NI];
  auto read_old = [&](auto vv_c) __attribute__((always_inline)) {
    constexpr int vv = decltype(vv_c)::value;
    const float* const rows = out + 16 * (wave * VTW + vv) * D;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      old[kEarly ? vv : 0][i] = *reinterpret_cast<const v4f*>(rows + (RPI * i + rsub) * D + 4 * c4);
  };
  if (kEarly && rmw) {
    read_old(IntC<0>{});
    if constexpr (VTW > 1) read_old(IntC<VTW - 1>{});
  }

  v4f acc[KT][VTW];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int vv = 0; vv < VTW; ++vv) acc[kt][vv] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t W = t1 - t0;
  const int64_t nchunks = (W + kC - 1) / kC;
  if (nchunks > 0) {
    // The head's gate parameters into LDS (read by every staging), while
    // the first chunk's inputs are in flight.
    if (!kAlpha && tid < (kChan ? D : 1)) {
      sh.PA[tid] = a.gate_expA[task.param_off + tid];
      sh.PD[tid] = a.gate_dt[task.param_off + tid];
    }
    if (tid < 64) sh.T[tid >> 3][8 + (tid & 7)] = 0.f;  // T12 of every chunk's inverse
    fetch(0);
    __syncthreads();
    stage1(0);
    if constexpr (!ONE) {
      if (nchunks > 1) fetch(1);
    }
    __syncthreads();
    stage2(0);
    __syncthreads();
    // ONE: the window bounds W by the task's window, at most kC, so the loop
    // runs once
    for (int64_t n = 0; n < nchunks; ++n) {
      const int cb = ONE ? 0 : static_cast<int>(n & 1), nb = cb ^ 1;
      // ---- phase 1: T(n), U0 = S Q(n)  ||  stage chunk n + 1, fetch n + 2
      if (wave == static_cast<int>(n % Sh::kNW)) invert();  // one wave, rotating
      v4f U[VTW];
#pragma unroll
      for (int vv = 0; vv < VTW; ++vv) U[vv] = v4f{0.f, 0.f, 0.f, 0.f};
      if (ONE || n == 0) {
        // the scratch state starts at zero: U0 = 0
      } else if constexpr (Sh::kSplit) {
        // K slots of lane group g: 4 g + e of k tile 2p (e < 4), then of
        // tile 2p + 1, on both operands.
#pragma unroll
        for (int kp = 0; kp < KT / 2; ++kp) {
          const uint32_t* qh0 = reinterpret_cast<const uint32_t*>(&sh.qw.Qh[m][32 * kp + 4 * g]);
          const uint32_t* qh1 = reinterpret_cast<const uint32_t*>(&sh.qw.Qh[m][32 * kp + 16 + 4 * g]);
          const uint32_t* ql0 = reinterpret_cast<const uint32_t*>(&sh.qw.Ql[m][32 * kp + 4 * g]);
          const uint32_t* ql1 = reinterpret_cast<const uint32_t*>(&sh.qw.Ql[m][32 * kp + 16 + 4 * g]);
          const u32x4 ah = {qh0[0], qh0[1], qh1[0], qh1[1]};
          const u32x4 al = {ql0[0], ql0[1], ql1[0], ql1[1]};
#pragma unroll
          for (int vv = 0; vv < VTW; ++vv) {
            const v4f x0 = acc[2 * kp][vv], x1 = acc[2 * kp + 1][vv];
            const u32x4 bh = {pack_bf16(hi_bits(x0[0]), hi_bits(x0[1])),
                              pack_bf16(hi_bits(x0[2]), hi_bits(x0[3])),
                              pack_bf16(hi_bits(x1[0]), hi_bits(x1[1])),
                              pack_bf16(hi_bits(x1[2]), hi_bits(x1[3]))};
            const u32x4 bl = {pack_bf16(lo_bits(x0[0]), lo_bits(x0[1])),
                              pack_bf16(lo_bits(x0[2]), lo_bits(x0[3])),
                              pack_bf16(lo_bits(x1[0]), lo_bits(x1[1])),
                              pack_bf16(lo_bits(x1[2]), lo_bits(x1[3]))};
            U[vv] = mfma_bf16(ah, bh, U[vv]);
            U[vv] = mfma_bf16(ah, bl, U[vv]);
            U[vv] = mfma_bf16(al, bh, U[vv]);
          }
        }
      } else {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const v4f qa = *reinterpret_cast<const v4f*>(&sh.qw.Q[m][16 * kt + 4 * g]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int vv = 0; vv < VTW; ++vv) U[vv] = mfma4(qa[r], acc[kt][vv][r], U[vv]);
        }
      }
      // staging and fetches past the request's last chunk are skipped
      if constexpr (!ONE) {
        if (n + 1 < nchunks) stage1(nb);
        if (n + 2 < nchunks) fetch(n + 2);
      }
      __syncthreads();
      // ---- phase 2: R, C = T R, S <- S Diag(gamma) + W C  ||  L, Q, W of n + 1
      {
        const v4f b4 = *reinterpret_cast<const v4f*>(&sh.B[cb][4 * g]);
        const v4f ta = *reinterpret_cast<const v4f*>(&sh.T[m][4 * g]);
        v4f Cc[VTW];
#pragma unroll
        for (int vv = 0; vv < VTW; ++vv) {
          const int v = 16 * (wave * VTW + vv) + m;
          v4f R;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            R[r] = b4[r] * (__uint_as_float(uint32_t(sh.V[cb][4 * g + r][v]) << 16) - U[vv][r]);
          Cc[vv] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int r = 0; r < 4; ++r) Cc[vv] = mfma4(ta[r], R[r], Cc[vv]);
        }
        if constexpr (Sh::kSplit) {
          // K slots of lane group g: token 4 g + e with W hi (e < 4) and
          // with W lo (e >= 4) on the A side; the B side is C hi for both
          // in the first product, and C lo against W hi (W lo against 0)
          // in the second.
          u32x4 chh[VTW], cl0[VTW];
#pragma unroll
          for (int vv = 0; vv < VTW; ++vv) {
            const uint32_t h0 = pack_bf16(hi_bits(Cc[vv][0]), hi_bits(Cc[vv][1]));
            const uint32_t h1 = pack_bf16(hi_bits(Cc[vv][2]), hi_bits(Cc[vv][3]));
            chh[vv] = u32x4{h0, h1, h0, h1};
            cl0[vv] = u32x4{pack_bf16(lo_bits(Cc[vv][0]), lo_bits(Cc[vv][1])),
                            pack_bf16(lo_bits(Cc[vv][2]), lo_bits(Cc[vv][3])), 0u, 0u};
          }
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const u32x4 wa = *reinterpret_cast<const u32x4*>(&sh.qw.W[cb][16 * kt + m][8 * g]);
#pragma unroll
            for (int vv = 0; vv < VTW; ++vv) {
              v4f x = acc[kt][vv];
              if constexpr (!ONE) {
                const v4f g4 = *reinterpret_cast<const v4f*>(&sh.G[cb][16 * kt + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] *= g4[r];
              }
              x = mfma_bf16(wa, chh[vv], x);
              x = mfma_bf16(wa, cl0[vv], x);
              acc[kt][vv] = x;
            }
          }
        } else {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const v4f wa = *reinterpret_cast<const v4f*>(&sh.qw.W[cb][16 * kt + m][4 * g]);
#pragma unroll
            for (int vv = 0; vv < VTW; ++vv) {
              v4f x = acc[kt][vv];
              if constexpr (!ONE) {
                const v4f g4 = *reinterpret_cast<const v4f*>(&sh.G[cb][16 * kt + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] *= g4[r];
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) x = mfma4(wa[r], Cc[vv][r], x);
              acc[kt][vv] = x;
            }
          }
        }
      }
      if constexpr (!ONE) {
        if (n + 1 < nchunks) stage2_waves(nb);
        __syncthreads();
      }
    }
  }

  // Write back the local units only ([dasc] §4.2).  Lane (g, m) of tile
  // (kt, vt) holds S[v][k .. k + 3] with v = 16 vt + m, k = 16 kt + 4 g.
  if constexpr (FUSED) {
    // Whole rows: retained column c of the head is unit j = (retained
    // channels below c) in the slot, D floats each from pool_off.  All the
    // gathers are issued before any store (the slot and the destination are
    // different buffers, which the compiler cannot know).
    const float* units = reinterpret_cast<const float*>(a.pool + slot * a.pool_stride +
                                                        task.pool_off);
    v4f y[KT][VTW];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const int k0 = 16 * kt + 4 * g;
      const int w = k0 >> 5, sh5 = k0 & 31;
      const uint32_t lw = w == 0 ? task.local[0] : w == 1 ? task.local[1]
                        : w == 2 ? task.local[2] : task.local[3];
      const uint32_t r4 = ~(lw >> sh5) & 0xFu;  // retained columns k0 .. k0 + 3
      uint32_t below = __popc(~lw & ((1u << sh5) - 1u));
#pragma unroll
      for (int q = 0; q < 3; ++q)
        if (q < w) below += __popc(~task.local[q]);
#pragma unroll
      for (int vv = 0; vv < VTW; ++vv) {
        const int v = 16 * (wave * VTW + vv) + m;
        y[kt][vv] = acc[kt][vv];
        uint32_t j = below;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if ((r4 >> c) & 1u) {
            y[kt][vv][c] = units[j * D + v];
            ++j;
          }
        }
      }
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int vv = 0; vv < VTW; ++vv)
        *reinterpret_cast<v4f*>(out + (16 * (wave * VTW + vv) + m) * D + 16 * kt + 4 * g) =
            y[kt][vv];
    return;
  }
  // The local columns are strided in the row-major state.  Each wave stages
  // one 16-row tile at a time in LDS (the staging buffers are dead by now)
  // and writes it row by row, lane c taking channel c (and c + 64): one
  // store instruction covers 64 consecutive channels of a row (two 128-byte
  // lines) with the local columns as its lane mask, where the tile layout
  // would spread a masked store over 16 rows.
  //
  // A store that covers part of a 32-byte sector costs the memory a read and
  // a write of the sector.  Where that dominates (the windowed refresh, a
  // short replay per head) and the head also holds retained columns, the
  // tile is written as whole rows instead: lane (rsub, c4) reads channels
  // 4 c4 .. 4 c4 + 3 of every RPI-th row (16 bytes; issued before the tile
  // is staged), puts the local values in and writes the 16 bytes back, which
  // streams faster than the masked 4-byte stores (KDA windows 1.23 -> 1.12
  // ms).  The full-suffix refresh keeps the masked stores: its write-back is
  // a small part of a long replay, and waiting for the reads at the end of
  // every head cost it about 1%.
  constexpr int RS = D + 4;  // padded LDS row
  static_assert(sizeof(sh) >= sizeof(float) * Sh::kNW * 16 * RS, "write-back staging");
  float* const stage = reinterpret_cast<float*>(&sh) + wave * 16 * RS;
  constexpr int HC = (D + 63) / 64;
  bool mine[HC];
#pragma unroll
  for (int hc = 0; hc < HC; ++hc) {
    const int c = 64 * hc + lane;
    const int w = c >> 5;  // selects, not an index: task stays in registers
    const uint32_t lw = w == 0 ? task.local[0] : w == 1 ? task.local[1]
                      : w == 2 ? task.local[2] : task.local[3];
    mine[hc] = c < D && ((lw >> (c & 31)) & 1u);
  }
  const int lw_i = (4 * c4) >> 5;
  const uint32_t lw4 = lw_i == 0 ? task.local[0] : lw_i == 1 ? task.local[1]
                     : lw_i == 2 ? task.local[2] : task.local[3];
  const uint32_t m4 = (lw4 >> ((4 * c4) & 31)) & 0xFu;  // the lane's local channels of 4 c4 ..
  auto write_tile = [&](auto vv_c) __attribute__((always_inline)) {
    constexpr int vv = decltype(vv_c)::value;  // a constant: acc stays in registers
    constexpr int ov = kEarly ? vv : 0;
    float* const rows = out + 16 * (wave * VTW + vv) * D;
    if (!kEarly && rmw) read_old(vv_c);
    __syncthreads();  // the previous tile's rows (or the last chunk's operands) are read
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
      *reinterpret_cast<v4f*>(&stage[m * RS + 16 * kt + 4 * g]) = acc[kt][vv];
    __syncthreads();
    if (rmw) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = RPI * i + rsub;
        v4f x = *reinterpret_cast<const v4f*>(&stage[r * RS + 4 * c4]);
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = (m4 >> c) & 1u ? x[c] : old[ov][i][c];
        *reinterpret_cast<v4f*>(rows + r * D + 4 * c4) = x;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int hc = 0; hc < HC; ++hc)
          if (mine[hc]) rows[r * D + 64 * hc + lane] = stage[r * RS + 64 * hc + lane];
      }
    }
  };
  write_tile(IntC<0>{});
  if constexpr (VTW > 1) write_tile(IntC<1>{});
  static_assert(VTW <= 2, "v tiles per wave");
}

// ---------------------------------------------------------------------------
// The same refresh in the recurrence's own form ([dasc] §3.1 Eq. 1), token
// by token, on the vector units: the reference point for the chunked
// kernel above (same inputs, same write-back, same tolerance).  One
// workgroup of 256 lanes per (head, request); lane (rb, cb) = (tid / 16,
// tid % 16) holds the B x B block of S (B = d / 16) in rows B rb .. and
// columns B cb ..; the 16 lanes of a DPP row share the rows, so
// u = S (alpha o k) is a B x B partial product per lane plus a 16-lane DPP
// sum.  Per token: u = S (alpha o k), c = beta (v - u), S <- S Diag(alpha)
// + c k^T.  Tokens are staged 16 at a time (decays by Eq. 2 from the gate
// logits) by the lanes that stage the chunked kernel's chunks.
// ---------------------------------------------------------------------------
template <int D, int GATE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
recurrent_kernel(RefreshArgs a) {
  constexpr int B = D / 16;
  constexpr int JB = D / 8;
  constexpr bool kChan = GATE != kGateHead;
  // k, decays and v of a batch of tokens; the write-back stages rows of the
  // state in the same memory
  __shared__ __attribute__((aligned(16))) float sKAV[3][kC][D];
  float(*const sK)[D] = sKAV[0];
  float(*const sA)[D] = sKAV[1];
  float(*const sV)[D] = sKAV[2];
  __shared__ float sB[kC];
  __shared__ float sPA[D], sPD[D];

  const RefreshTask task = a.tasks[blockIdx.x];
  const int req = blockIdx.y;
  const int64_t t0 = a.tok_off[req];
  const int64_t t1 = a.tok_off[req + 1];
  const int64_t dst = a.dst_idx[req];
  if (t0 < 0 || t1 < t0 || t1 > a.n_tokens) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, DASC_STATUS_BAD_TOKENS);
    return;
  }
  if (!in_range(dst, a.n_dense)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag(a.status, DASC_STATUS_BAD_INDEX);
    return;
  }
  const int tid = threadIdx.x;
  const int rb = tid / 16, cb = tid % 16;
  const int r0 = B * rb, c0 = B * cb;
  // staged item of this lane: token it_t of a batch, channels j0 .. j0 + 7
  const bool it_on = tid < 2 * D;
  const int it_t = (tid / JB) % kC, j0 = 8 * (tid % JB);

  if (tid < (kChan ? D : 1)) {
    sPA[tid] = a.gate_expA[task.param_off + tid];
    sPD[tid] = a.gate_dt[task.param_off + tid];
  }
  float S[B][B];
#pragma unroll
  for (int r = 0; r < B; ++r)
#pragma unroll
    for (int c = 0; c < B; ++c) S[r][c] = 0.f;

  const int64_t W = t1 - t0;
  for (int64_t n0 = 0; n0 < W; n0 += kC) {
    __syncthreads();  // the previous batch's reads (and the gate parameters)
    if (it_on) {
      const int64_t tok = t0 + n0 + it_t;
      const bool real = tok < t1;
      const int64_t tc = real ? tok : t1 - 1;  // in bounds; replaced below
      const u32x4 rk = *reinterpret_cast<const u32x4*>(a.k + tc * a.k_row + task.k_off + j0);
      const u32x4 rv = *reinterpret_cast<const u32x4*>(a.v + tc * a.v_row + task.v_off + j0);
      const uint16_t* ap = a.a + tc * a.g_row + task.g_off;
      float al[8];
      if constexpr (GATE == kGateHead) {
        const float x = decay(__uint_as_float(uint32_t(ap[0]) << 16) + sPD[0], sPA[0]);
#pragma unroll
        for (int c = 0; c < 8; ++c) al[c] = x;
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          al[c] = decay(__uint_as_float(uint32_t(ap[j0 + c]) << 16) + sPD[j0 + c], sPA[j0 + c]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sK[it_t][j0 + 2 * q] = real ? bf16_lo(rk[q]) : 0.f;
        sK[it_t][j0 + 2 * q + 1] = real ? bf16_hi(rk[q]) : 0.f;
        sV[it_t][j0 + 2 * q] = real ? bf16_lo(rv[q]) : 0.f;
        sV[it_t][j0 + 2 * q + 1] = real ? bf16_hi(rv[q]) : 0.f;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) sA[it_t][j0 + c] = real ? al[c] : 1.f;
      if (tid % JB == 0) sB[it_t] = real ? a.beta[tc * a.b_row + task.b_off] : 0.f;
    }
    __syncthreads();
    const int nt = static_cast<int>(W - n0 < kC ? W - n0 : kC);
    for (int i = 0; i < nt; ++i) {
      float al[B], kk[B], ak[B], u[B];
#pragma unroll
      for (int c = 0; c < B; ++c) {
        al[c] = sA[i][c0 + c];
        kk[c] = sK[i][c0 + c];
        ak[c] = al[c] * kk[c];
      }
#pragma unroll
      for (int r = 0; r < B; ++r) {
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < B; ++c) x = fmaf(S[r][c], ak[c], x);
        u[r] = group_sum<16>(x);
      }
      const float bt = sB[i];
#pragma unroll
      for (int r = 0; r < B; ++r) {
        const float cr = bt * (sV[i][r0 + r] - u[r]);
#pragma unroll
        for (int c = 0; c < B; ++c) S[r][c] = fmaf(cr, kk[c], S[r][c] * al[c]);
      }
    }
  }

  // The local columns of the head ([dasc] §4.2), as in the chunked kernel:
  // RP rows at a time staged in LDS, then stored row by row, lane t taking
  // channel t % D, so that one store instruction covers consecutive
  // channels of a row with the local columns as its lane mask.
  float* out = reinterpret_cast<float*>(a.dense + dst * a.dense_stride + task.dense_off);
  constexpr int RS = D + 4, RP = D < 32 ? D : 32;
  static_assert(RP * RS <= 3 * kC * D && kThreads % D == 0, "write-back staging");
  float* const stage = &sKAV[0][0][0];
  const int ch = tid % D;
  const int w = ch >> 5;  // selects, not an index: task stays in registers
  const uint32_t lw = w == 0 ? task.local[0] : w == 1 ? task.local[1]
                    : w == 2 ? task.local[2] : task.local[3];
  const bool mine = (lw >> (ch & 31)) & 1u;
#pragma unroll
  for (int p0 = 0; p0 < D; p0 += RP) {
    __syncthreads();  // the last batch's reads, or the previous rows' stores
    if (r0 >= p0 && r0 < p0 + RP) {
#pragma unroll
      for (int r = 0; r < B; ++r)
#pragma unroll
        for (int c = 0; c < B; ++c) stage[(r0 - p0 + r) * RS + c0 + c] = S[r][c];
    }
    __syncthreads();
    static_assert((RP * D) % kThreads == 0, "whole store rounds");
#pragma unroll
    for (int j = 0; j < RP * D / kThreads; ++j) {
      const int row = (tid + j * kThreads) / D;
      if (mine) out[(p0 + row) * D + ch] = stage[row * RS + ch];
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
bool kda_shape_supported(int d_k, int d_v) {
  return d_k >= 4 && d_v >= 4 && d_k <= 128 && d_v <= 128 && d_k % 4 == 0 && d_v % 4 == 0;
}

namespace {

// One launch of a mover over the pairs of `args`.
void launch_move_part(bool pack, const MoveArgs& args, hipStream_t s, size_t lds) {
  dim3 grid(args.n_pieces, static_cast<uint32_t>(args.n));
  const bool alt = args.tp;
  if (pack) {
    if (alt) {
      if (args.kda_128) move_kernel<true, 128, 128, true><<<grid, kThreads, lds, s>>>(args);
      else move_kernel<true, 0, 0, true><<<grid, kThreads, lds, s>>>(args);
    } else {
      if (args.kda_128) move_kernel<true, 128, 128, false><<<grid, kThreads, lds, s>>>(args);
      else move_kernel<true, 0, 0, false><<<grid, kThreads, lds, s>>>(args);
    }
  } else {
    if (alt) {
      if (args.kda_128) move_kernel<false, 128, 128, true><<<grid, kThreads, lds, s>>>(args);
      else move_kernel<false, 0, 0, true><<<grid, kThreads, lds, s>>>(args);
    } else {
      if (args.kda_128) move_kernel<false, 128, 128, false><<<grid, kThreads, lds, s>>>(args);
      else move_kernel<false, 0, 0, false><<<grid, kThreads, lds, s>>>(args);
    }
  }
}

void launch_qmove_part(bool pack, const MoveArgs& args, hipStream_t s) {
  dim3 grid(args.n_pieces, static_cast<uint32_t>(args.n));
  if (pack && args.q_blocks) qmove_kernel<true, true><<<grid, kThreads, 0, s>>>(args);
  else if (pack) qmove_kernel<true><<<grid, kThreads, 0, s>>>(args);
  else qmove_kernel<false><<<grid, kThreads, 0, s>>>(args);
}

// The pairs of a call, `per` at a time (more when a launch of `per` pairs
// would hold fewer than min_groups workgroups): the index arrays advance,
// every other argument stays.
template <typename F>
int by_pairs(const MoveArgs& args, int per, F&& launch, int64_t min_groups = kMinLaunchGroups) {
  per = mover_pairs_per_launch(args.n, args.n_pieces, per, min_groups);
  MoveArgs part = args;
  for (int32_t i = 0; i < args.n; i += per) {
    part.n = args.n - i < per ? args.n - i : per;
    part.src_idx = args.src_idx + i;
    part.dst_idx = args.dst_idx + i;
    if (args.alt_idx) part.alt_idx = args.alt_idx + i;
    launch(part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  return hipSuccess;
}

}  // namespace

int launch_move(bool pack, const MoveArgs& args, void* stream) {
  if (args.n == 0 || args.n_pieces == 0) return hipSuccess;
  if (args.n < 0 || args.n_pieces > 0x7FFFFFFFu || args.kda_r_max < 0 || args.kda_r_max > 128)
    return static_cast<int>(hipErrorInvalidValue);
  if (args.alt_base && !args.alt_idx) return static_cast<int>(hipErrorInvalidValue);
  const size_t lds = static_cast<size_t>(args.kda_r_max) * kKdaLdsRow * sizeof(float);  // <= 18 KiB
  hipStream_t s = static_cast<hipStream_t>(stream);
  return by_pairs(args, kMovePairs,
                  [&](const MoveArgs& part) { launch_move_part(pack, part, s, lds); });
}

int launch_qmove(bool pack, const MoveArgs& args, void* stream) {
  if (args.n == 0 || args.n_pieces == 0) return hipSuccess;
  if (args.n < 0 || args.n_pieces > 0x7FFFFFFFu) return static_cast<int>(hipErrorInvalidValue);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return by_pairs(
      args, pack ? kQPackPairs : kMovePairs,
      [&](const MoveArgs& part) { launch_qmove_part(pack, part, s); },
      pack ? kQPackMinGroups : kMinLaunchGroups);
}

bool refresh_shape_supported(int d_k, int d_v) {
  return d_k == d_v && (d_k == 16 || d_k == 32 || d_k == 64 || d_k == 128);
}

template <int D, int GATE, bool W>
void launch_refresh_f(const RefreshArgs& args, dim3 grid, hipStream_t s) {
  constexpr int kNT = RefreshShape<D>::kNT;
  if constexpr (W) {
    if (args.one_chunk) {
      if (args.pool) refresh_kernel<D, GATE, true, true, true><<<grid, kNT, 0, s>>>(args);
      else refresh_kernel<D, GATE, true, false, true><<<grid, kNT, 0, s>>>(args);
      return;
    }
  }
  if (args.pool) refresh_kernel<D, GATE, W, true, false><<<grid, kNT, 0, s>>>(args);
  else refresh_kernel<D, GATE, W, false, false><<<grid, kNT, 0, s>>>(args);
}

// Decays given as fp32 (no fused-load form).
template <int D, int GATE, bool W>
void launch_refresh_alpha_f(const RefreshArgs& args, dim3 grid, hipStream_t s) {
  constexpr int kNT = RefreshShape<D>::kNT;
  if (W && args.one_chunk) refresh_kernel<D, GATE, true, false, true><<<grid, kNT, 0, s>>>(args);
  else refresh_kernel<D, GATE, W, false, false><<<grid, kNT, 0, s>>>(args);
}

template <int D>
int launch_refresh_d(int gate, const RefreshArgs& args, dim3 grid, hipStream_t s) {
  const bool w = args.head_windows != 0;
  if (args.alpha) {
    if (args.pool) return static_cast<int>(hipErrorInvalidValue);
    switch (alpha_gate(gate)) {
      case kGateAlphaHead:
        if (w) launch_refresh_alpha_f<D, kGateAlphaHead, true>(args, grid, s);
        else launch_refresh_alpha_f<D, kGateAlphaHead, false>(args, grid, s);
        break;
      case kGateAlphaChan:
        if (w) launch_refresh_alpha_f<D, kGateAlphaChan, true>(args, grid, s);
        else launch_refresh_alpha_f<D, kGateAlphaChan, false>(args, grid, s);
        break;
      case kGateAlphaChanSplit:
        if (w) launch_refresh_alpha_f<D, kGateAlphaChanSplit, true>(args, grid, s);
        else launch_refresh_alpha_f<D, kGateAlphaChanSplit, false>(args, grid, s);
        break;
      default:
        return static_cast<int>(hipErrorInvalidValue);
    }
    return static_cast<int>(hipGetLastError());
  }
  switch (gate) {
    case kGateHead:
      if (w) launch_refresh_f<D, kGateHead, true>(args, grid, s);
      else launch_refresh_f<D, kGateHead, false>(args, grid, s);
      break;
    case kGateChan:
      if (w) launch_refresh_f<D, kGateChan, true>(args, grid, s);
      else launch_refresh_f<D, kGateChan, false>(args, grid, s);
      break;
    case kGateChanSplit:
      if (w) launch_refresh_f<D, kGateChanSplit, true>(args, grid, s);
      else launch_refresh_f<D, kGateChanSplit, false>(args, grid, s);
      break;
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

template <int D>
int launch_recurrent_d(int gate, const RefreshArgs& args, dim3 grid, hipStream_t s) {
  switch (gate) {
    case kGateHead: recurrent_kernel<D, kGateHead><<<grid, kThreads, 0, s>>>(args); break;
    case kGateChan: recurrent_kernel<D, kGateChan><<<grid, kThreads, 0, s>>>(args); break;
    case kGateChanSplit: recurrent_kernel<D, kGateChanSplit><<<grid, kThreads, 0, s>>>(args); break;
    default: return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

int launch_recurrent(int d, int gate, const RefreshArgs& args, void* stream) {
  if (args.n_tasks == 0 || args.n == 0) return hipSuccess;
  if (args.alpha) return static_cast<int>(hipErrorInvalidValue);  // gate logits only
  dim3 grid(args.n_tasks, static_cast<uint32_t>(args.n));
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 16: return launch_recurrent_d<16>(gate, args, grid, s);
    case 32: return launch_recurrent_d<32>(gate, args, grid, s);
    case 64: return launch_recurrent_d<64>(gate, args, grid, s);
    case 128: return launch_recurrent_d<128>(gate, args, grid, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

int launch_refresh(int d, int gate, const RefreshArgs& args, void* stream) {
  if (args.n_tasks == 0 || args.n == 0) return hipSuccess;
  dim3 grid(args.n_tasks, static_cast<uint32_t>(args.n));
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 16: return launch_refresh_d<16>(gate, args, grid, s);
    case 32: return launch_refresh_d<32>(gate, args, grid, s);
    case 64: return launch_refresh_d<64>(gate, args, grid, s);
    case 128: return launch_refresh_d<128>(gate, args, grid, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace dasc
