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
// Appendix B).  LDS holds one head, transposed: row k of T is column k of S.
// A lane moves 4x4 blocks: four 16-byte row loads, an in-register transpose,
// four 16-byte LDS stores (and the reverse for unpack).  LDS rows are
// rotated by whole 16-byte groups so that neither the block stores nor the
// row reads pile onto the same banks.
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct KdaShape {
  static constexpr int kLds = (DK && DV) ? DK * DV : 128 * 128;
};

__device__ __forceinline__ int rot(int g, int by, int groups) {
  int x = g + by;
  return x >= groups ? x - groups : x;  // by < groups, g < groups
}

template <int DK, int DV>
__global__ void __launch_bounds__(kThreads)
kda_pack_kernel(const KdaTask* __restrict__ tasks, const uint8_t* __restrict__ maps,
                const int32_t* __restrict__ src_idx, const int32_t* __restrict__ dst_idx,
                const uint8_t* __restrict__ src_base, int64_t src_stride, int64_t n_src,
                uint8_t* __restrict__ dst_base, int64_t dst_stride, int64_t n_dst,
                uint32_t* __restrict__ status, int dk_rt, int dv_rt) {
  __shared__ __attribute__((aligned(16))) float T[KdaShape<DK, DV>::kLds];
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
  const float* S = reinterpret_cast<const float*>(src_base + s * src_stride + t.dense_off);
  // Phase 1: whole head into LDS, transposed.
#pragma unroll 4
  for (int b = tid; b < NB; b += kThreads) {
    const int kg = b % KG, vg = b / KG;
    f32x4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = ld_stream(reinterpret_cast<const f32x4*>(S + (4 * vg + i) * dk + 4 * kg));
    const int pg = rot(vg, kg % VG, VG);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 col = {x[0][j], x[1][j], x[2][j], x[3][j]};
      *reinterpret_cast<f32x4*>(&T[(4 * kg + j) * dv + 4 * pg]) = col;
    }
  }
  __syncthreads();
  // Phase 2: retained columns, each one contiguous unit of d_v floats.
  const uint8_t* ret = maps + static_cast<uint64_t>(t.map_idx) * kMapBytes;
  float* P = reinterpret_cast<float*>(dst_base + d * dst_stride + t.pool_off);
  const int total = static_cast<int>(t.r) * VG;
  for (int q = tid; q < total; q += kThreads) {
    const int j = q / VG, g = q % VG;
    const int k = ret[j];
    const f32x4 val = *reinterpret_cast<const f32x4*>(&T[k * dv + 4 * rot(g, (k / 4) % VG, VG)]);
    st_stream(val, reinterpret_cast<f32x4*>(P + j * dv + 4 * g));
  }
}

template <int DK, int DV>
__global__ void __launch_bounds__(kThreads)
kda_unpack_kernel(const KdaTask* __restrict__ tasks, const uint8_t* __restrict__ maps,
                  const int32_t* __restrict__ src_idx, const int32_t* __restrict__ dst_idx,
                  const uint8_t* __restrict__ src_base, int64_t src_stride, int64_t n_src,
                  uint8_t* __restrict__ dst_base, int64_t dst_stride, int64_t n_dst,
                  uint32_t* __restrict__ status, int dk_rt, int dv_rt) {
  __shared__ __attribute__((aligned(16))) float U[KdaShape<DK, DV>::kLds];
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
// Eq. 1 in rank-1 form: with A = S Diag(alpha_t),
//   S_t = A + beta_t (v_t - A k_t) k_t^T,
// so per token each state element takes one multiply (decay), one FMA
// (the readout A k_t) and one FMA (the rank-1 write).  A lane owns 4 rows x
// 16 columns of S; the D/16 lanes that share rows sit next to each other and
// finish A k_t with DPP butterflies.  Tokens are staged through LDS in
// blocks of kTB (double-buffered): k, v widened from bf16, beta, and the
// decay alpha = exp(-exp(A_log) softplus(a_t + dt_bias)) (Eq. 2), each
// computed once per (token, channel).
// ---------------------------------------------------------------------------
constexpr int kTB = 16;

template <int D>
struct RefreshShape {
  static constexpr int kG = D / 16;             // lanes per row group
  static constexpr int kNS = D * D / 64;        // lanes that hold state
  static constexpr int kNT = kNS < 64 ? 64 : kNS;
  static constexpr int kPer = kTB * D / kNT;    // staged entries per lane per block
  static_assert(kNT % D == 0, "staging assumes a fixed channel per lane");
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

__device__ __forceinline__ float softplus_f32(float x) {
  return x > 20.f ? x : log1pf(expf(x));
}

template <int D>
__global__ void __launch_bounds__(RefreshShape<D>::kNT)
refresh_kernel(RefreshArgs a) {
  using Sh = RefreshShape<D>;
  constexpr int G = Sh::kG, NS = Sh::kNS, NT = Sh::kNT;
  __shared__ __attribute__((aligned(16))) float sA[2][kTB][D];
  __shared__ __attribute__((aligned(16))) float sK[2][kTB][D];
  __shared__ __attribute__((aligned(16))) float sV[2][kTB][D];
  __shared__ float sB[2][kTB];

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

  // Staging: lane `tid` always handles channel jj of tokens tid/D + m*NT/D.
  const int jj = tid % D;
  const bool kda = t.kind == static_cast<uint32_t>(kKDA);
  const uint32_t pidx = t.param_off + (kda ? jj : 0);
  const float expA = a.gate_expA[pidx];
  const float dtb = a.gate_dt[pidx];
  const int64_t gcol = t.g_off + (kda ? jj : 0);
  const int64_t kcol = t.k_off + jj;
  const int64_t vcol = t.v_off + jj;

  auto stage = [&](int buf, int64_t tok0, int nt) {
#pragma unroll
    for (int m = 0; m < Sh::kPer; ++m) {
      const int tt = tid / D + m * (NT / D);
      if (tt < nt) {
        const int64_t tok = tok0 + tt;
        const float x = bf16_to_f32(a.a[tok * a.g_row + gcol]) + dtb;
        sA[buf][tt][jj] = expf(-expA * softplus_f32(x));
        sK[buf][tt][jj] = bf16_to_f32(a.k[tok * a.k_row + kcol]);
        sV[buf][tt][jj] = bf16_to_f32(a.v[tok * a.v_row + vcol]);
        if (jj == 0) sB[buf][tt] = a.beta[tok * a.b_row + t.b_off];
      }
    }
  };

  float S[4][16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 16; ++c) S[i][c] = 0.f;

  const int64_t W = t1 - t0;
  const int64_t nb = (W + kTB - 1) / kTB;
  if (nb > 0) stage(0, t0, static_cast<int>(W < kTB ? W : kTB));
  __syncthreads();
  for (int64_t b = 0; b < nb; ++b) {
    const int buf = static_cast<int>(b & 1);
    const int64_t left = W - b * kTB;
    const int nt = static_cast<int>(left < kTB ? left : kTB);
    if (b + 1 < nb) {
      const int64_t left2 = left - kTB;
      stage(buf ^ 1, t0 + (b + 1) * kTB, static_cast<int>(left2 < kTB ? left2 : kTB));
    }
    if (has_state) {
      for (int tt = 0; tt < nt; ++tt) {
        float al[16], kk[16], vv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sA[buf][tt][c0 + 4 * q]);
          const f32x4 y = *reinterpret_cast<const f32x4*>(&sK[buf][tt][c0 + 4 * q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            al[4 * q + e] = x[e];
            kk[4 * q + e] = y[e];
          }
        }
        {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sV[buf][tt][r0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = x[e];
        }
        const float beta = sB[buf][tt];
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            S[i][c] *= al[c];                 // A = S Diag(alpha_t)
            acc = fmaf(S[i][c], kk[c], acc);  // (A k_t), partial over 16 columns
          }
          p[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = group_sum<G>(p[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ci = beta * (vv[i] - p[i]);  // beta_t (v_t - A k_t)
#pragma unroll
          for (int c = 0; c < 16; ++c) S[i][c] = fmaf(ci, kk[c], S[i][c]);
        }
      }
    }
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

int launch_kda(bool pack, int d_k, int d_v, const KdaTask* tasks, uint32_t n_tasks,
               const uint8_t* maps, const int32_t* src_idx, const int32_t* dst_idx,
               const uint8_t* src_base, int64_t src_stride, int64_t n_src, uint8_t* dst_base,
               int64_t dst_stride, int64_t n_dst, int32_t n, uint32_t* status, void* stream) {
  if (n_tasks == 0 || n == 0) return hipSuccess;
  if (!kda_shape_supported(d_k, d_v)) return static_cast<int>(hipErrorInvalidValue);
  dim3 grid(n_tasks, static_cast<uint32_t>(n));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fixed = d_k == 128 && d_v == 128;
  if (pack) {
    if (fixed)
      kda_pack_kernel<128, 128><<<grid, kThreads, 0, s>>>(tasks, maps, src_idx, dst_idx, src_base,
                                                          src_stride, n_src, dst_base, dst_stride,
                                                          n_dst, status, d_k, d_v);
    else
      kda_pack_kernel<0, 0><<<grid, kThreads, 0, s>>>(tasks, maps, src_idx, dst_idx, src_base,
                                                      src_stride, n_src, dst_base, dst_stride,
                                                      n_dst, status, d_k, d_v);
  } else {
    if (fixed)
      kda_unpack_kernel<128, 128><<<grid, kThreads, 0, s>>>(tasks, maps, src_idx, dst_idx,
                                                            src_base, src_stride, n_src, dst_base,
                                                            dst_stride, n_dst, status, d_k, d_v);
    else
      kda_unpack_kernel<0, 0><<<grid, kThreads, 0, s>>>(tasks, maps, src_idx, dst_idx, src_base,
                                                        src_stride, n_src, dst_base, dst_stride,
                                                        n_dst, status, d_k, d_v);
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
      refresh_kernel<16><<<grid, RefreshShape<16>::kNT, 0, s>>>(args);
      break;
    case 32:
      refresh_kernel<32><<<grid, RefreshShape<32>::kNT, 0, s>>>(args);
      break;
    case 64:
      refresh_kernel<64><<<grid, RefreshShape<64>::kNT, 0, s>>>(args);
      break;
    case 128:
      refresh_kernel<128><<<grid, RefreshShape<128>::kNT, 0, s>>>(args);
      break;
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace dasc
