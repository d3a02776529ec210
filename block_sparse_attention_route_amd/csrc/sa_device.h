// Device-side building blocks shared by the kernels of libsa_route:
// vector types, bf16/fp8 conversions, LDS swizzles, the float32 routing
// routine and small wave/workgroup reductions.  gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_layout.h"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
// proxy_row_pair() evaluates p_IJ = scale * (qbar_I . kbar_J) for one or two
// query blocks against every key block J in float32, in one fixed order:
// 16 lanes share a key row, lane j of the 16 accumulates dims
// [j*D/16, (j+1)*D/16) with sequential fmaf, then a fixed xor-tree over the
// 16 lanes.  The values therefore do not depend on how many waves run it, and
// the standalone route kernel and the fused attention kernel, which both call
// this routine, obtain identical bits.
//
// qbar: LDS, [2][D] (row 1 ignored when two == false).  kbar: global [Nb][D].
// p: LDS, [2][Nb] output.  Returns nothing; p is complete after a barrier.
// ---------------------------------------------------------------------------
template <int D, int NTHREADS>
__device__ __forceinline__ void proxy_row_pair(const float* __restrict__ qbar,
                                               const float* __restrict__ kbar, int Nb,
                                               float scale, bool two, float* __restrict__ p) {
  constexpr int DPL = D / 16;  // dims per lane
  const int tid = threadIdx.x;
  const int sub = tid & 15;
  const int slot = tid >> 4;
  constexpr int ROWS_PER_PASS = NTHREADS / 16;
  float q0[DPL], q1[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    q0[e] = qbar[sub * DPL + e];
    q1[e] = two ? qbar[D + sub * DPL + e] : 0.f;
  }
  for (int J0 = 0; J0 < Nb; J0 += ROWS_PER_PASS) {
    const int J = J0 + slot;
    float a0 = 0.f, a1 = 0.f;
    if (J < Nb) {
      const f32x4* row = reinterpret_cast<const f32x4*>(kbar + (size_t)J * D + sub * DPL);
#pragma unroll
      for (int e4 = 0; e4 < DPL / 4; ++e4) {
        f32x4 kv = row[e4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a0 = fmaf(q0[e4 * 4 + e], kv[e], a0);
          a1 = fmaf(q1[e4 * 4 + e], kv[e], a1);
        }
      }
    }
    // fixed xor tree over the 16 lanes that share row J
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      a0 = a0 + __shfl_xor(a0, off);
      a1 = a1 + __shfl_xor(a1, off);
    }
    if (J < Nb && sub == 0) {
      p[J] = a0 * scale;
      if (two) p[Nb + J] = a1 * scale;
    }
  }
}

// Row maxima of p (one or two rows) and the keep flags
// flags[J] = (p[0][J] >= m0 - tau) | (p[1][J] >= m1 - tau) << 1, plus the
// kept count of each row.  red: LDS scratch of >= 2*NTHREADS/64 floats and
// ints.  Requires a barrier between proxy_row_pair() and this call; ends
// with the flags, counts[2] complete (after the final barrier inside).
template <int NTHREADS>
__device__ __forceinline__ void threshold_rows(const float* __restrict__ p, int Nb, bool two,
                                               float tau, uint8_t* __restrict__ flags,
                                               float* __restrict__ redf, int* __restrict__ redi,
                                               int* __restrict__ counts) {
  constexpr int NW = NTHREADS / 64;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  float m0 = kNegInf, m1 = kNegInf;
  for (int J = tid; J < Nb; J += NTHREADS) {
    m0 = fmaxf(m0, p[J]);
    if (two) m1 = fmaxf(m1, p[Nb + J]);
  }
  m0 = wave_max(m0);
  m1 = wave_max(m1);
  if (lane == 0) {
    redf[wave] = m0;
    redf[NW + wave] = m1;
  }
  __syncthreads();
  m0 = redf[0];
  m1 = redf[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    m0 = fmaxf(m0, redf[w]);
    m1 = fmaxf(m1, redf[NW + w]);
  }
  const float thr0 = m0 - tau;
  const float thr1 = m1 - tau;
  int c0 = 0, c1 = 0;
  for (int J = tid; J < Nb; J += NTHREADS) {
    const int k0 = p[J] >= thr0 ? 1 : 0;
    const int k1 = (two && p[Nb + J] >= thr1) ? 1 : 0;
    flags[J] = (uint8_t)(k0 | (k1 << 1));
    c0 += k0;
    c1 += k1;
  }
  c0 = wave_sum_int(c0);
  c1 = wave_sum_int(c1);
  if (lane == 0) {
    redi[wave] = c0;
    redi[NW + wave] = c1;
  }
  __syncthreads();
  if (tid == 0) {
    int s0 = 0, s1 = 0;
    for (int w = 0; w < NW; ++w) {
      s0 += redi[w];
      s1 += redi[NW + w];
    }
    counts[0] = s0;
    counts[1] = s1;
  }
  __syncthreads();
}

// XCD-aware tile order: workgroups are handed to the 8 XCDs round-robin, so
// workgroup w runs on XCD w % 8.  Give each XCD one contiguous range of tiles
// (adjacent query blocks of the same head share key blocks in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int w, int G) {
  const int q = G >> 3, r = G & 7;
  const int x = w & 7, i = w >> 3;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace sa
