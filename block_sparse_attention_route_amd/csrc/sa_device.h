// Device-side building blocks shared by the kernels of libsa_route:
// vector types, bf16/fp8 conversions, LDS swizzles, the float32 routing
// routine and small wave/workgroup reductions.  gfx950 (CDNA4, wave64) only.
#pragma once
#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_layout.h"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 (finite inputs), via the gfx950
// conversion instruction that the __bf16 cast lowers to.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// OCP e4m3fn byte -> float (exact).  Bias 7, no infinities, 0x7f/0xff = NaN
// (never produced by the input quantiser).
__device__ __forceinline__ float fp8e4m3_to_f32(uint32_t byte) {
  uint32_t s = (byte & 0x80u) << 24;
  uint32_t e = (byte >> 3) & 0xFu;
  uint32_t m = byte & 0x7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;  // m * 2^-9 (subnormal)
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return __uint_as_float(__float_as_uint(mag) | s);
}

// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (one query per lane column),
// followed by O^T = V^T P^T: if MFMA row m of a 32-key tile reads key row
// kperm(m) (bits 2 and 3 swapped), the keys a lane holds in its S^T
// accumulators are exactly the keys of its B operand in the PV product.
__device__ __forceinline__ int kperm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Key (within a 32-key tile) of accumulator element r of S^T, lane half h.
__device__ __forceinline__ int key_of(int r, int h) { return r < 8 ? 8 * h + r : 8 + 8 * h + r; }

// Position of a 16-byte chunk in an LDS row, XOR-swizzled so that 16 lanes
// reading the same logical chunk of 16 consecutive rows hit distinct banks.
// chunks_per_row is 16 (256-byte rows) or 8 (128-byte rows).
template <int CPR>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (CPR == 16) {
    return chunk ^ (row & 15);
  } else {
    static_assert(CPR == 8, "rows of 8 or 16 chunks");
    return chunk ^ ((row >> 1) & 7);
  }
}

// Sum over aligned groups of L lanes (L = 2, 4, 8 or 16; a group lies inside
// one 16-lane DPP row), every lane of a group receiving the same bits: pairs
// (i, i^1), then (i, i^2) by quad permutation, then mirrored half-rows
// (i, 7-i) and rows (i, 15-i).  Each step adds two equal-shaped partial sums
// symmetrically, so the order is fixed and lane-independent; all on the
// vector ALU (no LDS permute).
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(L == 2 || L == 4 || L == 8 || L == 16, "group of 2..16 lanes");
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});                       // quad_perm [1,0,3,2]
  if constexpr (L >= 4) x += dpp(x, std::integral_constant<int, 0x4E>{});  // quad_perm [2,3,0,1]
  if constexpr (L >= 8) x += dpp(x, std::integral_constant<int, 0x141>{}); // row_half_mirror
  if constexpr (L >= 16) x += dpp(x, std::integral_constant<int, 0x140>{}); // row_mirror
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// ---------------------------------------------------------------------------
// Routing (Sol-Attn page, "Abstract": query-dependent threshold on a pooled
// score, selected on chip without materialising a proxy map).
//
// proxy_rows() evaluates p_IJ = scale * (qbar_I . kbar_J) for QB query blocks
// against every key block J in float32, in one fixed order: 16 lanes share a
// key row, lane j of the 16 accumulates dims [j*D/16, (j+1)*D/16) with
// sequential fmaf, then group_sum over the 16 lanes.  The value of a
// pair (I, J) therefore does not depend on QB or on the number of threads, so
// the standalone route kernel and every attention kernel, which all call this
// routine, obtain identical bits.
//
// qbar: LDS [QB][D] (rows >= nrows ignored).  kbar: global [Nb][D].
// p: LDS [QB][Nb] output, complete after a barrier.  tid: the thread index
// in the workgroup (as do the routines below).
// ---------------------------------------------------------------------------
template <int D, int NTHREADS, int QB>
__device__ __forceinline__ void proxy_rows(const float* __restrict__ qbar,
                                           const float* __restrict__ kbar, int Nb, float scale,
                                           int nrows, float* __restrict__ p, int tid) {
  constexpr int DPL = D / 16;  // dims per lane
  const int sub = tid & 15;
  const int slot = tid >> 4;
  constexpr int ROWS_PER_PASS = NTHREADS / 16;
  float qv[QB][DPL];
#pragma unroll
  for (int r = 0; r < QB; ++r)
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[r][e] = (r < nrows) ? qbar[r * D + sub * DPL + e] : 0.f;
  // U passes at a time, their loads issued together (the key means come
  // from L2 or beyond; one pass at a time would wait out that latency U times)
  constexpr int U = 4;
  for (int J0 = 0; J0 < Nb; J0 += ROWS_PER_PASS * U) {
    f32x4 kv[U][DPL / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int J = J0 + u * ROWS_PER_PASS + slot;
      const f32x4* row = reinterpret_cast<const f32x4*>(kbar + (size_t)(J < Nb ? J : 0) * D + sub * DPL);
#pragma unroll
      for (int e4 = 0; e4 < DPL / 4; ++e4) kv[u][e4] = row[e4];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int J = J0 + u * ROWS_PER_PASS + slot;
      float acc[QB];
#pragma unroll
      for (int r = 0; r < QB; ++r) acc[r] = 0.f;
#pragma unroll
      for (int e4 = 0; e4 < DPL / 4; ++e4)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int r = 0; r < QB; ++r) acc[r] = fmaf(qv[r][e4 * 4 + e], kv[u][e4][e], acc[r]);
      // fixed-order sum over the 16 lanes that share row J
#pragma unroll
      for (int r = 0; r < QB; ++r) acc[r] = group_sum<16>(acc[r]);
      if (J < Nb && sub == 0) {
#pragma unroll
        for (int r = 0; r < QB; ++r)
          if (r < nrows) p[r * Nb + J] = acc[r] * scale;
      }
    }
  }
}

// Row maxima of the first nrows rows of p and the keep flags
// flags[J] = OR over rows r of [p[r][J] >= m_r - tau] << r, plus the kept
// count of each row in counts[r].  redf, redi: LDS scratch of QB*NTHREADS/64
// entries.  Needs a barrier between proxy_rows() and this call; ends with a
// barrier after which flags and counts are complete.
template <int NTHREADS, int QB>
__device__ __forceinline__ void threshold_rows(const float* __restrict__ p, int Nb, int nrows,
                                               float tau, uint8_t* __restrict__ flags,
                                               float* __restrict__ redf, int* __restrict__ redi,
                                               int* __restrict__ counts, int tid) {
  constexpr int NW = NTHREADS / 64;
  const int wave = tid >> 6, lane = tid & 63;
  float m[QB];
#pragma unroll
  for (int r = 0; r < QB; ++r) m[r] = kNegInf;
  for (int J = tid; J < Nb; J += NTHREADS)
#pragma unroll
    for (int r = 0; r < QB; ++r)
      if (r < nrows) m[r] = fmaxf(m[r], p[r * Nb + J]);
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    m[r] = wave_max(m[r]);
    if (lane == 0) redf[r * NW + wave] = m[r];
  }
  __syncthreads();
  float thr[QB];
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    float mm = redf[r * NW];
#pragma unroll
    for (int w = 1; w < NW; ++w) mm = fmaxf(mm, redf[r * NW + w]);
    thr[r] = mm - tau;
  }
  int c[QB];
#pragma unroll
  for (int r = 0; r < QB; ++r) c[r] = 0;
  for (int J = tid; J < Nb; J += NTHREADS) {
    int f = 0;
#pragma unroll
    for (int r = 0; r < QB; ++r) {
      const int k = (r < nrows && p[r * Nb + J] >= thr[r]) ? 1 : 0;
      f |= k << r;
      c[r] += k;
    }
    flags[J] = (uint8_t)f;
  }
#pragma unroll
  for (int r = 0; r < QB; ++r) {
    c[r] = wave_sum_int(c[r]);
    if (lane == 0) redi[r * NW + wave] = c[r];
  }
  __syncthreads();
  if (tid < QB) {
    int sum = 0;
    for (int w = 0; w < NW; ++w) sum += redi[tid * NW + w];
    counts[tid] = sum;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Fixed-budget routing (the paper review of the Sol Video Inference Engine,
// xllm-io blog, runs PISA at block size 64 and a fixed sparsity): row r keeps
// the min(topk, Nb) key blocks of largest p[r][.], equal values in increasing
// J.  The kept set is a function of the float32 values alone, so every caller
// obtains the same set.  It is found by a radix select over order-preserving
// 32-bit keys, most significant byte first (4 histogram passes), which
// yields the k-th largest key T and how many blocks equal to T are kept; a
// tie at T that is only partly kept is resolved by the rank among equal keys.
//
// p: LDS [QB][Nb] after a barrier.  hist: LDS [QB][256] ints.  sel: LDS
// [3*QB] uint32 (key prefix, remaining count, count equal to T).  wsum: LDS
// [QB * NTHREADS/64] ints.  Writes flags[J] (bit r) and counts[r]; ends with
// a barrier.  Needs NTHREADS/64 >= QB.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0: equal values, equal keys
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NTHREADS, int QB>
__device__ __forceinline__ void topk_rows(const float* __restrict__ p, int Nb, int nrows, int topk,
                                          uint8_t* __restrict__ flags, int* __restrict__ hist,
                                          uint32_t* __restrict__ sel, int* __restrict__ wsum,
                                          int* __restrict__ counts, int tid) {
  constexpr int NW = NTHREADS / 64;
  static_assert(NW >= QB, "one wave per row for the digit search");
  const int wave = tid >> 6, lane = tid & 63;
  const int kk = min(topk, Nb);
  uint32_t* prefix = sel;            // [QB] key bits fixed so far
  uint32_t* need = sel + QB;         // [QB] blocks still to take among those matching prefix
  uint32_t* neq = sel + 2 * QB;      // [QB] blocks whose key equals T
  if (tid < QB) {
    prefix[tid] = 0u;
    need[tid] = (uint32_t)kk;
    neq[tid] = 0u;
  }
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t himask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < QB * 256; i += NTHREADS) hist[i] = 0;
    __syncthreads();
    for (int J = tid; J < Nb; J += NTHREADS)
#pragma unroll
      for (int r = 0; r < QB; ++r)
        if (r < nrows) {
          const uint32_t key = order_key(p[r * Nb + J]);
          if ((key & himask) == (prefix[r] & himask)) atomicAdd(&hist[r * 256 + ((key >> shift) & 255u)], 1);
        }
    __syncthreads();
    if (wave < nrows) {
      // lane l holds bins 4l .. 4l+3; find the bin holding the need-th largest
      const int r = wave;
      int c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[r * 256 + 4 * lane + j];
      const int own = c[0] + c[1] + c[2] + c[3];
      int suffix = own;  // sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_down(suffix, off);
        if (lane + off < 64) suffix += y;
      }
      const int above = suffix - own;
      const int nd = (int)need[r];
      if (above < nd && nd <= suffix) {
        int cum = above;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (cum + c[j] >= nd) {
            prefix[r] |= (uint32_t)(4 * lane + j) << shift;
            need[r] = (uint32_t)(nd - cum);
            neq[r] = (uint32_t)c[j];
            break;
          }
          cum += c[j];
        }
      }
    }
    __syncthreads();
  }
  bool partial = false;  // some row keeps only part of a tie at T
#pragma unroll
  for (int r = 0; r < QB; ++r)
    if (r < nrows && need[r] < neq[r]) partial = true;
  if (!partial) {
    for (int J = tid; J < Nb; J += NTHREADS) {
      int f = 0;
#pragma unroll
      for (int r = 0; r < QB; ++r)
        if (r < nrows && order_key(p[r * Nb + J]) >= prefix[r]) f |= 1 << r;
      flags[J] = (uint8_t)f;
    }
  } else {
    // contiguous segments per thread, exclusive scan of the count of keys
    // equal to T: a block equal to T is kept iff fewer than need[r] equal
    // blocks precede it
    const int seg = (Nb + NTHREADS - 1) / NTHREADS;
    const int j0 = min(Nb, tid * seg), j1 = min(Nb, j0 + seg);
    int cnt[QB];
#pragma unroll
    for (int r = 0; r < QB; ++r) {
      cnt[r] = 0;
      if (r < nrows)
        for (int j = j0; j < j1; ++j) cnt[r] += order_key(p[r * Nb + j]) == prefix[r];
    }
    int incl[QB];
#pragma unroll
    for (int r = 0; r < QB; ++r) {
      int x = cnt[r];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      incl[r] = x;
      if (lane == 63) wsum[r * NW + wave] = x;
    }
    __syncthreads();
    int rank[QB];
#pragma unroll
    for (int r = 0; r < QB; ++r) {
      int base = 0;
      for (int w = 0; w < wave; ++w) base += wsum[r * NW + w];
      rank[r] = base + incl[r] - cnt[r];
    }
    for (int j = j0; j < j1; ++j) {
      int f = 0;
#pragma unroll
      for (int r = 0; r < QB; ++r) {
        if (r >= nrows) continue;
        const uint32_t key = order_key(p[r * Nb + j]);
        if (key > prefix[r]) {
          f |= 1 << r;
        } else if (key == prefix[r]) {
          if (rank[r] < (int)need[r]) f |= 1 << r;
          ++rank[r];
        }
      }
      flags[j] = (uint8_t)f;
    }
  }
  if (tid < QB) counts[tid] = tid < nrows ? kk : 0;
  __syncthreads();
}

#ifndef SA_XCD_CHUNK
#define SA_XCD_CHUNK 64
#endif
#ifndef SA_XCD_CHUNK_SPARSE
#define SA_XCD_CHUNK_SPARSE 16
#endif

// XCD-aware tile order.  Workgroups are handed to the 8 XCDs round-robin, so
// workgroup w runs on XCD w % 8 as that XCD's (w / 8)-th workgroup.  Tiles
// are cut into chunks of CH consecutive tiles (adjacent query blocks of one
// head) and chunk c goes to XCD c % 8: the workgroups resident on one XCD
// share key blocks in its L2, and all eight XCDs stay on the same head at a
// time, so the head's K/V stays resident in the shared last-level cache.
// Dense workgroups all cost the same and take chunks of about what an XCD
// holds at once (SA_XCD_CHUNK); sparse ones differ in cost with the kept
// density of their region, and smaller chunks (SA_XCD_CHUNK_SPARSE) spread
// each region over the XCDs before an XCD that runs out of its own groups
// takes those of the others.
// CH = 0 keeps the plain order.  Tiles past the last whole round keep their
// own index.
template <int CH>
__device__ __forceinline__ int xcd_remap(int w, int G) {
  if constexpr (CH == 0) {
    return w;
  } else {
    const int full = G / (8 * CH) * (8 * CH);
    if (w >= full) return w;
    const int x = w & 7, i = w >> 3;
    return (i / CH) * (8 * CH) + x * CH + (i % CH);
  }
}

}  // namespace sa
