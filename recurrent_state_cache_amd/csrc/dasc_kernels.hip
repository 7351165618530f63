// HIP kernels for gfx950 (CDNA4, wave64) of the dasc checkpoint hot path.
//
// Pages cited by title:
//   [dasc] "dasc: Decay-Aware State Compression for Hybrid Linear-Attention
//          Serving" (arXiv HTML version): §3.1 Eq. 1, §3.3 Eq. 2, §4.1, §4.2,
//          Appendix B (ragged Scheme 2).
//
// Pack and unpack are pure data movement: every workgroup takes one task of
// the plan's lists for one (checkpoint, slot) pair and moves raw bits with
// 16-byte accesses.  KDA units are strided columns of a row-major state, so
// a KDA task stages its head through LDS as a 4x4-block register transpose.
// The refresh keeps one head's fp32 state resident in registers (4 rows x 16
// columns per lane) and replays Eq. 1 token by token.
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
// Contiguous ranges: GDN heads (whole-unit copies), conv bytes, and the
// zero-fill of omitted GDN heads / fully omitted KDA heads.
// pack:   src = dense checkpoint, dst = pool slot
// unpack: src = pool slot,        dst = dense checkpoint
// ---------------------------------------------------------------------------
template <bool kPack>
__global__ void __launch_bounds__(kThreads)
copy_kernel(const CopyTask* __restrict__ tasks, const int32_t* __restrict__ src_idx,
            const int32_t* __restrict__ dst_idx, const uint8_t* __restrict__ src_base,
            int64_t src_stride, int64_t n_src, uint8_t* __restrict__ dst_base,
            int64_t dst_stride, int64_t n_dst, uint32_t* __restrict__ status) {
  const CopyTask t = tasks[blockIdx.x];
  const int64_t s = src_idx[blockIdx.y];
  const int64_t d = dst_idx[blockIdx.y];
  if (!in_range(s, n_src) || !in_range(d, n_dst)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag(status, DASC_STATUS_BAD_INDEX);
    return;
  }
  const uint64_t src_off = kPack ? t.dense_off : t.pool_off;
  const uint64_t dst_off = kPack ? t.pool_off : t.dense_off;
  u32x4* dst = reinterpret_cast<u32x4*>(dst_base + d * dst_stride + dst_off);
  const uint32_t nv = t.bytes >> 4;
  const uint32_t tid = threadIdx.x;
  if (!kPack && t.type == kTaskZero) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (uint32_t i = tid; i < nv; i += kThreads) st_stream(z, dst + i);
    return;
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(src_base + s * src_stride + src_off);
  if (nv == kCopyChunk / 16) {
    // A full 64 KiB chunk: all 16 loads of a lane in flight before any store.
    constexpr int kPer = kCopyChunk / 16 / kThreads;
    u32x4 r[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) r[j] = ld_stream(src + tid + kThreads * j);
#pragma unroll
    for (int j = 0; j < kPer; ++j) st_stream(r[j], dst + tid + kThreads * j);
  } else {
    for (uint32_t i = tid; i < nv; i += kThreads) st_stream(ld_stream(src + i), dst + i);
  }
}

// ---------------------------------------------------------------------------
// KDA heads.  The state S is [d_v][d_k] row-major; the unit (h, k) is the
// column S[:, k], stored in the pool as d_v contiguous floats ([dasc] §4.1,
// Appendix B).  LDS holds only the head's r retained columns, as rows
// U[j][0..d_v) in pool order (j = rank of the channel among the retained
// ones), so its size is r_max * d_v floats for the task group instead of a
// whole head.  A lane moves 4x4 blocks of S: four 16-byte row accesses and an
// in-register transpose.  Each LDS row is rotated by whole 16-byte groups
// (by its row index) so that lanes touching different rows spread over the
// banks; lanes walking one row touch consecutive groups.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int rot(int g, int by, int groups) {
  int x = g + by;
  return x >= groups ? x - groups : x;  // by < groups, g < groups
}

// pack: dense head -> LDS (retained columns only) -> contiguous pool units
template <int DK, int DV>
__global__ void __launch_bounds__(kThreads)
kda_pack_kernel(const KdaTask* __restrict__ tasks, const uint8_t* __restrict__ maps,
                const int32_t* __restrict__ src_idx, const int32_t* __restrict__ dst_idx,
                const uint8_t* __restrict__ src_base, int64_t src_stride, int64_t n_src,
                uint8_t* __restrict__ dst_base, int64_t dst_stride, int64_t n_dst,
                uint32_t* __restrict__ status, int dk_rt, int dv_rt) {
  extern __shared__ __attribute__((aligned(16))) float U[];
  const int dk = DK ? DK : dk_rt;
  const int dv = DV ? DV : dv_rt;
  const KdaTask t = tasks[blockIdx.x];
  const int64_t s = src_idx[blockIdx.y];
  const int64_t d = dst_idx[blockIdx.y];
  if (!in_range(s, n_src) || !in_range(d, n_dst)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag(status, DASC_STATUS_BAD_INDEX);
    return;
  }
  const int KG = dk / 4, VG = dv / 4, NB = KG * VG;
  const int tid = threadIdx.x;
  const uint8_t* rank_of = maps + static_cast<uint64_t>(t.map_idx) * kMapBytes + 128;
  const float* S = reinterpret_cast<const float*>(src_base + s * src_stride + t.dense_off);
  // Phase 1: read the whole head (strided columns force whole rows), keep
  // the retained columns.
#pragma unroll 4
  for (int b = tid; b < NB; b += kThreads) {
    const int kg = b % KG, vg = b / KG;
    f32x4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = ld_stream(reinterpret_cast<const f32x4*>(S + (4 * vg + i) * dk + 4 * kg));
    const uint32_t ranks = *reinterpret_cast<const uint32_t*>(rank_of + 4 * kg);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t rk = (ranks >> (8 * c)) & 0xFFu;
      if (rk != kLocal) {
        f32x4 col = {x[0][c], x[1][c], x[2][c], x[3][c]};
        *reinterpret_cast<f32x4*>(&U[rk * dv + 4 * rot(vg, rk % VG, VG)]) = col;
      }
    }
  }
  __syncthreads();
  // Phase 2: the r units, contiguous in the pool slot.
  float* P = reinterpret_cast<float*>(dst_base + d * dst_stride + t.pool_off);
  const int total = static_cast<int>(t.r) * VG;
  for (int q = tid; q < total; q += kThreads) {
    const int j = q / VG, g = q % VG;
    const f32x4 val = *reinterpret_cast<const f32x4*>(&U[j * dv + 4 * rot(g, j % VG, VG)]);
    st_stream(val, reinterpret_cast<f32x4*>(P + j * dv + 4 * g));
  }
}

// unpack: contiguous pool units -> LDS -> every element of the dense head,
// +0.0 in omitted channels
template <int DK, int DV>
__global__ void __launch_bounds__(kThreads)
kda_unpack_kernel(const KdaTask* __restrict__ tasks, const uint8_t* __restrict__ maps,
                  const int32_t* __restrict__ src_idx, const int32_t* __restrict__ dst_idx,
                  const uint8_t* __restrict__ src_base, int64_t src_stride, int64_t n_src,
                  uint8_t* __restrict__ dst_base, int64_t dst_stride, int64_t n_dst,
                  uint32_t* __restrict__ status, int dk_rt, int dv_rt) {
  extern __shared__ __attribute__((aligned(16))) float U[];
  const int dk = DK ? DK : dk_rt;
  const int dv = DV ? DV : dv_rt;
  const KdaTask t = tasks[blockIdx.x];
  const int64_t s = src_idx[blockIdx.y];
  const int64_t d = dst_idx[blockIdx.y];
  if (!in_range(s, n_src) || !in_range(d, n_dst)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag(status, DASC_STATUS_BAD_INDEX);
    return;
  }
  const int KG = dk / 4, VG = dv / 4, NB = KG * VG;
  const int tid = threadIdx.x;
  // Phase 1: the head's r stored units (contiguous) into LDS rows j < r.
  const float* P = reinterpret_cast<const float*>(src_base + s * src_stride + t.pool_off);
  const int total = static_cast<int>(t.r) * VG;
  for (int q = tid; q < total; q += kThreads) {
    const int j = q / VG, g = q % VG;
    const f32x4 val = ld_stream(reinterpret_cast<const f32x4*>(P + j * dv + 4 * g));
    *reinterpret_cast<f32x4*>(&U[j * dv + 4 * rot(g, j % VG, VG)]) = val;
  }
  __syncthreads();
  // Phase 2: every element of the dense head; omitted channels get +0.0.
  const uint8_t* rank_of = maps + static_cast<uint64_t>(t.map_idx) * kMapBytes + 128;
  float* S = reinterpret_cast<float*>(dst_base + d * dst_stride + t.dense_off);
#pragma unroll 4
  for (int b = tid; b < NB; b += kThreads) {
    const int kg = b % KG, vg = b / KG;
    const uint32_t ranks = *reinterpret_cast<const uint32_t*>(rank_of + 4 * kg);
    f32x4 col[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t rk = (ranks >> (8 * c)) & 0xFFu;
      if (rk != kLocal) {
        col[c] = *reinterpret_cast<const f32x4*>(&U[rk * dv + 4 * rot(vg, rk % VG, VG)]);
      } else {
        col[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 row = {col[0][i], col[1][i], col[2][i], col[3][i]};
      st_stream(row, reinterpret_cast<f32x4*>(S + (4 * vg + i) * dk + 4 * kg));
    }
  }
}

// ---------------------------------------------------------------------------
// Bounded-suffix refresh ([dasc] §4.2), one workgroup per (head, request).
//
// Eq. 1 ([dasc] §3.1) is replayed in chunks of C tokens.  Inside a chunk
// that starts from S_0, with the running decay gamma_t = alpha_1 ... alpha_t
// and the pairwise decay D_{t,s} = alpha_{s+1} ... alpha_t (s < t), the
// recurrence unrolls exactly to
//   S_t = S_0 Diag(gamma_t) + sum_{s<=t} c_s (k_s o D_{t,s})^T,
//   c_t = beta_t (v_t - S_0 (gamma_t o k_t) - sum_{s<t} M_{t,s} c_s),
//   M_{t,s} = sum_j k_t[j] k_s[j] D_{t,s}[j],
// so a chunk costs one product S_0 Q (Q = [gamma_t o k_t]), a C x C
// forward substitution for the c_t, and one rank-C update
// S_C = S_0 Diag(gamma_C) + sum_s c_s (k_s o D_{C,s})^T: two FMAs per state
// element and token instead of a multiply and two FMAs, and every factor is a
// product of decays (no division, so fast-decaying channels cannot overflow).
// Tokens past the end of a request pad the last chunk as exact no-ops
// (alpha = 1, k = 0, v = 0, beta = 0).
//
// Lanes: each lane owns 4 rows x 16 columns of S; the D/16 lanes sharing rows
// are adjacent and finish the readout with DPP butterflies.  Chunk inputs are
// staged through LDS (double-buffered): the decay alpha = exp(-exp(A_log)
// softplus(a_t + dt_bias)) ([dasc] §3.3 Eq. 2) once per (token, channel),
// then gamma, Q, W = [k_s o D_{C,s}] and M.
// ---------------------------------------------------------------------------
template <int D, int C>
struct RefreshShape {
  static constexpr int kG = D / 16;             // lanes per row group
  static constexpr int kNS = D * D / 64;        // lanes that hold state
  static constexpr int kNT = kNS < 64 ? 64 : kNS;
  static constexpr int kPer = C * D / kNT;      // staged entries per lane per chunk
  static_assert(kNT % D == 0, "staging assumes a fixed channel per lane");
  static_assert(C * D % kNT == 0, "staging covers a chunk exactly");
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, true));
}

// Sum over the G consecutive lanes of a row group (G in {1, 2, 4, 8, 16}).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (G >= 16) x += dpp<0x140>(x); // row_mirror
  return x;
}

// alpha = exp(-exp(A_log) softplus(x)) with x = a_t + dt_bias (Eq. 2);
// expA = exp(A_log) is precomputed per unit.
__device__ __forceinline__ float decay(float x, float expA) {
  const float sp = fmaxf(x, 0.f) + log1pf(__builtin_amdgcn_exp2f(-fabsf(x) * 1.44269504088896341f));
  return __builtin_amdgcn_exp2f(-expA * sp * 1.44269504088896341f);
}

constexpr int kChunk = 8;

template <int D, int C>
__global__ void __launch_bounds__((RefreshShape<D, C>::kNT))
refresh_kernel(RefreshArgs a) {
  using Sh = RefreshShape<D, C>;
  constexpr int G = Sh::kG, NS = Sh::kNS, NT = Sh::kNT, PER = Sh::kPer;
  // per chunk (double-buffered): Q = gamma o k, W = k o D_{C,.}, v, gamma_C, beta, M
  __shared__ __attribute__((aligned(16))) float sQ[2][C][D];
  __shared__ __attribute__((aligned(16))) float sW[2][C][D];
  __shared__ __attribute__((aligned(16))) float sV[2][C][D];
  __shared__ __attribute__((aligned(16))) float sG[2][D];
  __shared__ float sB[2][C];
  __shared__ float sM[2][C][C];
  // staging scratch (single): k and alpha of the chunk being staged
  __shared__ __attribute__((aligned(16))) float sK[C][D];
  __shared__ __attribute__((aligned(16))) float sA[C][D];

  const RefreshTask t = a.tasks[blockIdx.x];
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
  const bool has_state = tid < NS;
  const int c0 = (tid % G) * 16;
  const int r0 = (tid / G) * 4;

  // Staging: lane `tid` handles channel jj of tokens tid/D + m*NT/D.
  const int jj = tid % D;
  const bool kda = t.kind == static_cast<uint32_t>(kKDA);
  const uint32_t pidx = t.param_off + (kda ? jj : 0);
  const float expA = a.gate_expA[pidx];
  const float dtb = a.gate_dt[pidx];
  const int64_t gcol = t.g_off + (kda ? jj : 0);
  const int64_t kcol = t.k_off + jj;
  const int64_t vcol = t.v_off + jj;

  const int64_t W = t1 - t0;
  const int64_t nchunks = (W + C - 1) / C;

  uint16_t ra[PER], rk[PER], rv[PER];
  float rb[PER];
  auto fetch = [&](int64_t n) {  // raw inputs of chunk n into registers
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int tt = tid / D + m * (NT / D);
      const int64_t tok = t0 + n * C + tt;
      if (tok < t1) {
        ra[m] = a.a[tok * a.g_row + gcol];
        rk[m] = a.k[tok * a.k_row + kcol];
        rv[m] = a.v[tok * a.v_row + vcol];
        rb[m] = jj == 0 ? a.beta[tok * a.b_row + t.b_off] : 0.f;
      } else {  // padding: an exact no-op step
        ra[m] = 0;
        rk[m] = 0;
        rv[m] = 0;
        rb[m] = 0.f;
      }
    }
  };
  auto stage_a = [&](int buf, int64_t n) {  // decay, k, v, beta
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int tt = tid / D + m * (NT / D);
      const bool real = t0 + n * C + tt < t1;
      sA[tt][jj] = real ? decay(bf16_to_f32(ra[m]) + dtb, expA) : 1.f;
      sK[tt][jj] = bf16_to_f32(rk[m]);
      sV[buf][tt][jj] = bf16_to_f32(rv[m]);
      if (jj == 0) sB[buf][tt] = rb[m];
    }
  };
  auto stage_b = [&](int buf) {  // gamma, Q, W, gamma_C and M from sK, sA
    for (int j = tid; j < D; j += NT) {
      float g = 1.f;
#pragma unroll
      for (int tt = 0; tt < C; ++tt) {
        g *= sA[tt][j];
        sQ[buf][tt][j] = g * sK[tt][j];
      }
      sG[buf][j] = g;
      float dd = 1.f;
#pragma unroll
      for (int s = C - 1; s >= 0; --s) {
        sW[buf][s][j] = sK[s][j] * dd;
        dd *= sA[s][j];
      }
    }
    if constexpr (D == 128 && NT == 256 && C == 8) {
      // threads 128..255: (token t, block of 8 channels); M_{t,s} summed
      // over the 16 blocks with DPP inside each 16-lane row
      if (tid >= 128) {
        const int u = tid - 128;
        const int tt = u >> 4, j0 = (u & 15) * 8;
        float p[8], kt[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) p[c] = kt[c] = sK[tt][j0 + c];
        (void)kt;
        for (int s = tt - 1; s >= 0; --s) {
          float part = 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            p[c] *= sA[s + 1][j0 + c];
            part = fmaf(p[c], sK[s][j0 + c], part);
          }
          part = group_sum<16>(part);
          if ((u & 15) == 0) sM[buf][tt][s] = part;
        }
      }
    } else {
      for (int e = tid; e < C * C; e += NT) {
        const int tt = e / C, s = e % C;
        if (s < tt) {
          float acc = 0.f;
          for (int j = 0; j < D; ++j) {
            float p = sK[tt][j];
            for (int r = s + 1; r <= tt; ++r) p *= sA[r][j];
            acc = fmaf(p, sK[s][j], acc);
          }
          sM[buf][tt][s] = acc;
        }
      }
    }
  };

  float S[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 16; ++c) S[i][c] = 0.f;

  if (nchunks > 0) {
    fetch(0);
    stage_a(0, 0);
  }
  __syncthreads();
  if (nchunks > 0) stage_b(0);
  __syncthreads();
  for (int64_t n = 0; n < nchunks; ++n) {
    const int b = static_cast<int>(n & 1);
    const bool more = n + 1 < nchunks;
    if (more) fetch(n + 1);
    if (has_state) {
      float U[4][C];
      // readout of the chunk-start state: U[i][t] = (S_0 q_t)_i
#pragma unroll
      for (int tt = 0; tt < C; ++tt) {
        float q[16];
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sQ[b][tt][c0 + 4 * v4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) q[4 * v4 + e] = x[e];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) acc = fmaf(S[i][c], q[c], acc);
          U[i][tt] = acc;
        }
      }
#pragma unroll
      for (int tt = 0; tt < C; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) U[i][tt] = group_sum<G>(U[i][tt]);
      // forward substitution: U[i][t] <- c_t for the lane's rows
#pragma unroll
      for (int tt = 0; tt < C; ++tt) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&sV[b][tt][r0]);
        const float beta = sB[b][tt];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = v[i] - U[i][tt];
#pragma unroll
          for (int s = 0; s < tt; ++s) x = fmaf(-sM[b][tt][s], U[i][s], x);
          U[i][tt] = beta * x;
        }
      }
      // S <- S Diag(gamma_C) + sum_s c_s w_s^T
      {
        float g[16];
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sG[b][c0 + 4 * v4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) g[4 * v4 + e] = x[e];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 16; ++c) S[i][c] *= g[c];
      }
#pragma unroll
      for (int s = 0; s < C; ++s) {
        float w[16];
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sW[b][s][c0 + 4 * v4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) w[4 * v4 + e] = x[e];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 16; ++c) S[i][c] = fmaf(U[i][s], w[c], S[i][c]);
      }
    }
    if (more) stage_a(b ^ 1, n + 1);
    __syncthreads();
    if (more) stage_b(b ^ 1);
    __syncthreads();
  }

  // Write back the local units only ([dasc] §4.2): whole GDN heads, or the
  // local columns of a KDA head.
  if (has_state) {
    float* out = reinterpret_cast<float*>(a.dense + dst * a.dense_stride + t.dense_off);
    // select the mask word without a dynamic index (keeps `t` in registers)
    const uint32_t lw = c0 < 32 ? t.local[0] : c0 < 64 ? t.local[1] : c0 < 96 ? t.local[2] : t.local[3];
    const uint32_t m16 = (lw >> (c0 & 31)) & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* row = out + (r0 + i) * D + c0;
      if (m16 == 0xFFFFu) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 x = {S[i][4 * q], S[i][4 * q + 1], S[i][4 * q + 2], S[i][4 * q + 3]};
          *reinterpret_cast<f32x4*>(row + 4 * q) = x;
        }
      } else if (m16 != 0u) {
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if ((m16 >> c) & 1u) row[c] = S[i][c];
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int launch_copy(bool pack, const CopyTask* tasks, uint32_t n_tasks, const int32_t* src_idx,
                const int32_t* dst_idx, const uint8_t* src_base, int64_t src_stride,
                int64_t n_src, uint8_t* dst_base, int64_t dst_stride, int64_t n_dst,
                int32_t n, uint32_t* status, void* stream) {
  if (n_tasks == 0 || n == 0) return hipSuccess;
  dim3 grid(n_tasks, static_cast<uint32_t>(n));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pack)
    copy_kernel<true><<<grid, kThreads, 0, s>>>(tasks, src_idx, dst_idx, src_base, src_stride,
                                                n_src, dst_base, dst_stride, n_dst, status);
  else
    copy_kernel<false><<<grid, kThreads, 0, s>>>(tasks, src_idx, dst_idx, src_base, src_stride,
                                                 n_src, dst_base, dst_stride, n_dst, status);
  return static_cast<int>(hipGetLastError());
}

bool kda_shape_supported(int d_k, int d_v) {
  return d_k >= 4 && d_v >= 4 && d_k <= 128 && d_v <= 128 && d_k % 4 == 0 && d_v % 4 == 0;
}

int launch_kda(bool pack, int d_k, int d_v, int r_max, const KdaTask* tasks, uint32_t n_tasks,
               const uint8_t* maps, const int32_t* src_idx, const int32_t* dst_idx,
               const uint8_t* src_base, int64_t src_stride, int64_t n_src, uint8_t* dst_base,
               int64_t dst_stride, int64_t n_dst, int32_t n, uint32_t* status, void* stream) {
  if (n_tasks == 0 || n == 0) return hipSuccess;
  if (!kda_shape_supported(d_k, d_v) || r_max < 1 || r_max > d_k)
    return static_cast<int>(hipErrorInvalidValue);
  dim3 grid(n_tasks, static_cast<uint32_t>(n));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t lds = static_cast<size_t>(r_max) * d_v * sizeof(float);  // <= 64 KiB
  const bool fixed = d_k == 128 && d_v == 128;
  if (pack) {
    if (fixed)
      kda_pack_kernel<128, 128><<<grid, kThreads, lds, s>>>(tasks, maps, src_idx, dst_idx,
                                                            src_base, src_stride, n_src, dst_base,
                                                            dst_stride, n_dst, status, d_k, d_v);
    else
      kda_pack_kernel<0, 0><<<grid, kThreads, lds, s>>>(tasks, maps, src_idx, dst_idx, src_base,
                                                        src_stride, n_src, dst_base, dst_stride,
                                                        n_dst, status, d_k, d_v);
  } else {
    if (fixed)
      kda_unpack_kernel<128, 128><<<grid, kThreads, lds, s>>>(tasks, maps, src_idx, dst_idx,
                                                              src_base, src_stride, n_src,
                                                              dst_base, dst_stride, n_dst, status,
                                                              d_k, d_v);
    else
      kda_unpack_kernel<0, 0><<<grid, kThreads, lds, s>>>(tasks, maps, src_idx, dst_idx,
                                                          src_base, src_stride, n_src, dst_base,
                                                          dst_stride, n_dst, status, d_k, d_v);
  }
  return static_cast<int>(hipGetLastError());
}

bool refresh_shape_supported(int d_k, int d_v) {
  return d_k == d_v && (d_k == 16 || d_k == 32 || d_k == 64 || d_k == 128);
}

int launch_refresh(int d, const RefreshArgs& args, void* stream) {
  if (args.n_tasks == 0 || args.n == 0) return hipSuccess;
  dim3 grid(args.n_tasks, static_cast<uint32_t>(args.n));
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d) {
    case 16:
      refresh_kernel<16, kChunk><<<grid, RefreshShape<16, kChunk>::kNT, 0, s>>>(args);
      break;
    case 32:
      refresh_kernel<32, kChunk><<<grid, RefreshShape<32, kChunk>::kNT, 0, s>>>(args);
      break;
    case 64:
      refresh_kernel<64, kChunk><<<grid, RefreshShape<64, kChunk>::kNT, 0, s>>>(args);
      break;
    case 128:
      refresh_kernel<128, kChunk><<<grid, RefreshShape<128, kChunk>::kNT, 0, s>>>(args);
      break;
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace dasc
