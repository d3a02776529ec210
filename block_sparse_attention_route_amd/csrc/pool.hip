// Step "pool": block means of Q, K, V (the operands of the pooled routing
// score and of the skipped-block correction), plus V regrouped per 64-key
// block for the attention kernels.
//
// The Sol-Attn project page (section "Abstract") routes on a pooled score;
// this library reads "pooled" as the mean over each 64-token block's actual
// tokens.  Blocks are taken over positions: the raster order, or the 3-D
// tile order of the token grid (sa_layout.h, token_of), in which case K is
// also written out in position order.  The kernel is HBM-bound: it reads Q, K
// and V once (each workgroup one 64-token block of one head, all three
// tensors in flight together; with the producer step one block position of
// up to eight heads, which share its rotation angles) and writes 1/16 as many
// bytes of means plus the regrouped V.
//
// With the producer step fused in front (ProArgs), the rows read are the raw
// Q/K projections: each is RMS-normalised over its D features, scaled by the
// gain, rotated pairwise by its 3-D position (frame, row and column groups of
// feature pairs), rounded to bf16, written to q_out / k_out, and pooled from
// the rounded values -- the same bits sa_pool would read back.  The paper
// review of the Sol Video Inference Engine (xllm-io blog) lists fused
// RoPE + norm and fused QK + RoPE among the fusions in front of attention.
//
// Every sum is taken in one fixed order (per-thread sequential over rows,
// then the partial sums of the row groups in order), so the means, and all
// routing decisions made from them, are bitwise reproducible.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {
namespace {

template <int E>
struct EltBytes;
template <>
struct EltBytes<ELT_F32> { static constexpr int v = 4; };
template <>
struct EltBytes<ELT_BF16> { static constexpr int v = 2; };
template <>
struct EltBytes<ELT_FP8> { static constexpr int v = 1; };

// A 64-token block read as 16-byte chunks by 256 threads: thread t owns
// chunk column c = t % CPR of rows g, g + G, ... with g = t / CPR.
template <int E, int D>
struct Tiling {
  static constexpr int B = EltBytes<E>::v;
  static constexpr int EPC = 16 / B;      // elements per chunk
  static constexpr int CPR = D * B / 16;  // chunks per row
  static constexpr int G = 256 / CPR;     // row groups
  static constexpr int P = kBlock / G;    // chunks per thread
};

template <int E>
__device__ __forceinline__ void unpack(const u32x4& c, float* out) {
  if constexpr (E == ELT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(c[i]);
  } else if constexpr (E == ELT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(c[i] << 16);
      out[2 * i + 1] = __uint_as_float(c[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[4 * i + j] = fp8e4m3_to_f32((c[i] >> (8 * j)) & 0xFFu);
  }
}

// Rows pos0 .. pos0 + nrows - 1 of the block, in position order: row r is
// token token_of(tm, pos0 + r) of the head whose tokens start at `head`.
template <int E, int D>
__device__ __forceinline__ void load_block(const uint8_t* __restrict__ head, int pos0, int nrows,
                                           const TileMap& tm, u32x4 (&raw)[Tiling<E, D>::P]) {
  using T = Tiling<E, D>;
  const int c = threadIdx.x % T::CPR, g = threadIdx.x / T::CPR;
#pragma unroll
  for (int i = 0; i < T::P; ++i) {
    const int r = g + T::G * i;
    raw[i] = u32x4{0u, 0u, 0u, 0u};
    if (r < nrows) {
      const size_t tok = (size_t)token_of(tm, pos0 + r);
      raw[i] = *reinterpret_cast<const u32x4*>(head + tok * D * T::B + c * 16);
    }
  }
}

// Per-thread sums over its rows (sequential, rows g, g+G, ...; absent rows
// hold zeros) -> acc.
template <int E, int D>
__device__ __forceinline__ void thread_sums(const u32x4 (&raw)[Tiling<E, D>::P], float (&acc)[Tiling<E, D>::EPC]) {
  using T = Tiling<E, D>;
#pragma unroll
  for (int e = 0; e < T::EPC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < T::P; ++i) {
    float x[T::EPC];
    unpack<E>(raw[i], x);
#pragma unroll
    for (int e = 0; e < T::EPC; ++e) acc[e] += x[e];
  }
}

// Per-thread sums -> mean over rows in out[0..D) (fp32), scaled by mult; the
// row groups' partial sums are added in order through part[G][D] in LDS.
// With out_bf16, the mean also goes out as two bf16 halves: hi = bf16(m) at
// out_bf16[d] and lo = bf16(m - hi) at out_bf16[lo_off + d] (hi + lo carries
// about 16 significant bits).
template <int E, int D>
__device__ __forceinline__ void mean_finish(const float (&acc)[Tiling<E, D>::EPC], int nrows, float mult,
                                            float* __restrict__ part, float* __restrict__ out_f32,
                                            uint16_t* __restrict__ out_bf16, size_t lo_off = 0) {
  using T = Tiling<E, D>;
  const int c = threadIdx.x % T::CPR, g = threadIdx.x / T::CPR;
#pragma unroll
  for (int e = 0; e < T::EPC; ++e) part[g * D + c * T::EPC + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float s = 0.f;
#pragma unroll
    for (int gg = 0; gg < T::G; ++gg) s += part[gg * D + d];
    const float m = (s / (float)nrows) * mult;
    out_f32[d] = m;
    if (out_bf16) {
      const uint16_t hi = f32_to_bf16_bits(m);
      out_bf16[d] = hi;
      out_bf16[lo_off + d] = f32_to_bf16_bits(m - bf16_bits_to_f32(hi));
    }
  }
  __syncthreads();
}

// mean over rows -> out[0..D) (fp32), scaled by mult; uses part[G][D] in LDS.
template <int E, int D>
__device__ __forceinline__ void block_mean(const u32x4 (&raw)[Tiling<E, D>::P], int nrows,
                                           float mult, float* __restrict__ part,
                                           float* __restrict__ out_f32,
                                           uint16_t* __restrict__ out_bf16, size_t lo_off = 0) {
  float acc[Tiling<E, D>::EPC];
  thread_sums<E, D>(raw, acc);
  mean_finish<E, D>(acc, nrows, mult, part, out_f32, out_bf16, lo_off);
}

// Rotation angles of this thread's rows: (cos, sin) of pos_a * theta for its
// four feature pairs, pairs split into consecutive frame / row / column
// groups of D - 4*(D/6), 2*(D/6), 2*(D/6) features and pair j of a group of
// d_a features turning at theta = base^(-2 j / d_a).  Thread (c, g) owns
// features 8c .. 8c+7 = pairs 4c .. 4c+3 of rows g, g+G, ...  The angles of
// a position are the same for every head, so a workgroup computes them once
// for all the heads it produces.
template <int D, int NP>
struct RopeRows {
  float cs[NP][4], sn[NP][4];
  int tok[NP];
};

template <int D, int NP>
__device__ __forceinline__ void rope_rows(int pos0, int nrows, const TileMap& tm, const ProArgs& pr,
                                          RopeRows<D, NP>& out) {
  using T = Tiling<ELT_BF16, D>;
  static_assert(NP == T::P, "rows per thread");
  const int c = threadIdx.x % T::CPR, g = threadIdx.x / T::CPR;
  constexpr int DY = 2 * (D / 6), DT = D - 2 * DY;
  float theta[4];
  int axis[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int f = 8 * c + 2 * q;  // first feature of the pair
    int j, da;
    if (f < DT) {
      axis[q] = 0; j = f / 2; da = DT;
    } else if (f < DT + DY) {
      axis[q] = 1; j = (f - DT) / 2; da = DY;
    } else {
      axis[q] = 2; j = (f - DT - DY) / 2; da = DY;
    }
    theta[q] = powf(pr.base, -2.0f * (float)j / (float)da);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = g + T::G * i;
    const int tok = token_of(tm, pos0 + (r < nrows ? r : 0));
    out.tok[i] = tok;
    const int pt = tok / (pr.Hg * pr.Wg), py = (tok / pr.Wg) % pr.Hg, px = tok % pr.Wg;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float pa = (float)(axis[q] == 0 ? pt : (axis[q] == 1 ? py : px));
      sincosf(pa * theta[q], &out.sn[i][q], &out.cs[i][q]);
    }
  }
}

// RMS norm + gain + rotation of this thread's rows of one tensor (Q or K),
// in place on the raw bf16 chunks, rounded to bf16; the rows are stored to
// out (token order) and their sums over the thread's rows returned in acc.  The CPR threads of a row are
// adjacent lanes.
template <int D, int NP>
__device__ __forceinline__ void norm_rope(u32x4 (&raw)[NP], int nrows, const float* __restrict__ gain,
                                          float eps, const RopeRows<D, NP>& ang, uint16_t* __restrict__ out,
                                          float (&acc)[8]) {
  using T = Tiling<ELT_BF16, D>;
  const int c = threadIdx.x % T::CPR, g = threadIdx.x / T::CPR;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float gv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gv[e] = gain[8 * c + e];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = g + T::G * i;
    float x[8];
    unpack<ELT_BF16>(raw[i], x);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss = group_sum<T::CPR>(ss);
    if (r >= nrows) continue;
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float cs = ang.cs[i][q], sn = ang.sn[i][q];
      const float u = x[2 * q] * inv * gv[2 * q], v = x[2 * q + 1] * inv * gv[2 * q + 1];
      w[q] = (uint32_t)f32_to_bf16_bits(u * cs - v * sn) | ((uint32_t)f32_to_bf16_bits(u * sn + v * cs) << 16);
    }
    raw[i] = w;
    *reinterpret_cast<u32x4*>(out + (size_t)ang.tok[i] * D + 8 * c) = w;
    // the block sums of the rounded values, in the order thread_sums takes
    // (absent rows would add +0, which leaves a sum started at +0 unchanged)
    float y[8];
    unpack<ELT_BF16>(w, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += y[e];
  }
}

// One 64-token block J of head bh: load, (producer step), means, V regrouped.
template <int QE, int VE, int D, bool VT_ONLY, bool PRO>
__device__ __forceinline__ void pool_block(const PoolArgs& a, int J, int bh, float* part, uint16_t* vtl,
                                           const RopeRows<D, Tiling<ELT_BF16, D>::P>* ang) {
  const int row0 = J * kBlock;
  const int nrows = min(kBlock, a.N - row0);
  const size_t head0 = (size_t)bh * a.N;
  using TQ = Tiling<QE, D>;
  using TV = Tiling<VE, D>;
  u32x4 rq[TQ::P], rk[TQ::P], rv[TV::P];
  const TileMap tm = a.tm;
  if constexpr (!VT_ONLY) {
    load_block<QE, D>(reinterpret_cast<const uint8_t*>(a.q) + head0 * D * TQ::B, row0, nrows, tm, rq);
    load_block<QE, D>(reinterpret_cast<const uint8_t*>(a.k) + head0 * D * TQ::B, row0, nrows, tm, rk);
  }
  load_block<VE, D>(reinterpret_cast<const uint8_t*>(a.v) + head0 * D * TV::B, row0, nrows, tm, rv);
  const size_t mrow = ((size_t)bh * a.Nb + J) * D;

  auto qk_part = [&]() {
    if constexpr (!VT_ONLY) {
      if constexpr (PRO) {
        // the producer writes Q/K in token order; the means come from the
        // rounded values
        static_assert(QE == ELT_BF16, "producer step on bf16 rows");
        float acc[8];
        norm_rope<D>(rq, nrows, a.pro.q_gain, a.pro.eps, *ang, a.pro.q_out + head0 * D, acc);
        mean_finish<QE, D>(acc, nrows, 1.f, part, a.qbar + mrow, nullptr);
        norm_rope<D>(rk, nrows, a.pro.k_gain, a.pro.eps, *ang, a.pro.k_out + head0 * D, acc);
        mean_finish<QE, D>(acc, nrows, 1.f, part, a.kbar + mrow, a.kbar16 + ((size_t)bh * a.Nbp + J) * D,
                           (size_t)a.BH * a.Nbp * D);
        if (tm.on) {
          // 3-D tile order: K also in position order
          const int c = threadIdx.x % TQ::CPR, g = threadIdx.x / TQ::CPR;
          uint8_t* dst = reinterpret_cast<uint8_t*>(a.kpos16) + (head0 + row0) * D * 2;
#pragma unroll
          for (int i = 0; i < TQ::P; ++i) {
            const int r = g + TQ::G * i;
            if (r < nrows)
              *reinterpret_cast<u32x4*>(dst + (size_t)r * D * 2 + c * 16) = rk[i];
          }
        }
        return;
      }
      if constexpr (QE == ELT_BF16) {
        // 3-D tile order: K also in position order, for the attention
        // kernel's contiguous tile copies
        if (tm.on) {
          const int c = threadIdx.x % TQ::CPR, g = threadIdx.x / TQ::CPR;
          uint8_t* dst = reinterpret_cast<uint8_t*>(a.kpos16) + (head0 + row0) * D * 2;
#pragma unroll
          for (int i = 0; i < TQ::P; ++i) {
            const int r = g + TQ::G * i;
            if (r < nrows) *reinterpret_cast<u32x4*>(dst + (size_t)r * D * 2 + c * 16) = rk[i];
          }
        }
      }
      float qm = 1.f, km = 1.f;
      if constexpr (QE == ELT_FP8) {
        qm = a.q_scale[(size_t)bh * a.Nb + J];
        km = a.k_scale[(size_t)bh * a.Nb + J];
      }
      block_mean<QE, D>(rq, nrows, qm, part, a.qbar + mrow, nullptr);
      uint16_t* k16 = (VE == ELT_BF16) ? a.kbar16 + ((size_t)bh * a.Nbp + J) * D : nullptr;
      block_mean<QE, D>(rk, nrows, km, part, a.kbar + mrow, k16, (size_t)a.BH * a.Nbp * D);
    }
  };

  auto v_part = [&]() {
    if constexpr (!VT_ONLY) block_mean<VE, D>(rv, nrows, 1.f, part, a.vbar + mrow, nullptr);
    if constexpr (VE == ELT_BF16) {
      // V^T of this block into LDS: element (d, r) at row d, 16-byte chunk
      // (r/8) ^ ((d/8) & 7), slot r % 8 (rows are 64 keys = 128 bytes).
      const int c = threadIdx.x % TV::CPR, g = threadIdx.x / TV::CPR;
#pragma unroll
      for (int i = 0; i < TV::P; ++i) {
        const int r = g + TV::G * i;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = c * 8 + e;
          const uint32_t word = rv[i][e >> 1];
          const uint16_t val = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFFu);
          const int pc = (r >> 3) ^ ((d >> 3) & 7);
          vtl[d * kBlock + pc * 8 + (r & 7)] = val;
        }
      }
      __syncthreads();
      uint8_t* dst = reinterpret_cast<uint8_t*>(a.vt16 + ((size_t)bh * a.Nb + J) * D * kBlock);
      constexpr int NCH = D * kBlock * 2 / 16;  // 16-byte chunks in the tile
#pragma unroll
      for (int x = threadIdx.x; x < NCH; x += 256) {
        const int d = x >> 3, cc = x & 7;
        const int pc = cc ^ ((d >> 3) & 7);
        *reinterpret_cast<u32x4*>(dst + (size_t)x * 16) =
            *reinterpret_cast<const u32x4*>(&vtl[d * kBlock + pc * 8]);
      }
      if constexpr (!VT_ONLY) {
        // bf16(vbar) into the transposed groups of 64 blocks.
        if (threadIdx.x < D) {
          const int d = threadIdx.x;
          const size_t grp = (size_t)bh * (a.Nbp / 64) + (J >> 6);
          a.vbarT16[(grp * D + d) * 64 + (J & 63)] = f32_to_bf16_bits(a.vbar[mrow + d]);
        }
        // the last block of a head zero-fills the padding up to Nbp
        if (J == a.Nb - 1) {
          for (int JJ = a.Nb; JJ < a.Nbp; ++JJ) {
            if (threadIdx.x < D) {
              const int d = threadIdx.x;
              a.kbar16[((size_t)bh * a.Nbp + JJ) * D + d] = 0;
              a.kbar16[((size_t)(a.BH + bh) * a.Nbp + JJ) * D + d] = 0;
              const size_t grp = (size_t)bh * (a.Nbp / 64) + (JJ >> 6);
              a.vbarT16[(grp * D + d) * 64 + (JJ & 63)] = 0;
            }
          }
        }
      }
      // vtl is rewritten by the next head's block
      __syncthreads();
    }
  };

  qk_part();
  v_part();
}

#ifndef SA_PRO_HEADS
#define SA_PRO_HEADS 8
#endif
// heads per workgroup of the producer step (they share the rotation angles)
constexpr int kProHeads = SA_PRO_HEADS;

template <int QE, int VE, int D, bool VT_ONLY, bool PRO>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  __shared__ float part[4096];  // up to 64 row groups x 64 dims or 32 x 128
  __shared__ __attribute__((aligned(16))) uint16_t vtl[D * kBlock];
  const int J = blockIdx.x;
  // the attention kernel's group counters start zeroed (its launcher zeroes
  // them again before every launch), so the pool leaves no byte of the
  // workspace undefined
  if (!VT_ONLY && a.sched && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) a.sched[threadIdx.x] = 0;
  if constexpr (PRO) {
    RopeRows<D, Tiling<ELT_BF16, D>::P> ang;
    rope_rows<D>(J * kBlock, min(kBlock, a.N - J * kBlock), a.tm, a.pro, ang);
    const int bh0 = blockIdx.y * kProHeads;
    const int bh1 = min(bh0 + kProHeads, a.BH);
    for (int bh = bh0; bh < bh1; ++bh) pool_block<QE, VE, D, VT_ONLY, true>(a, J, bh, part, vtl, &ang);
  } else {
    pool_block<QE, VE, D, VT_ONLY, false>(a, J, blockIdx.y, part, vtl, nullptr);
  }
}

template <int QE, int VE, int D>
hipError_t launch_t(const PoolArgs& a, hipStream_t st) {
  dim3 grid(a.Nb, a.BH);
  if (a.vt_only) {
    if constexpr (VE == ELT_BF16) {
      hipLaunchKernelGGL((pool_kernel<QE, VE, D, true, false>), grid, dim3(256), 0, st, a);
    } else {
      return hipSuccess;
    }
  } else if (a.pro.on) {
    if constexpr (QE == ELT_BF16) {
      const dim3 pgrid(a.Nb, (a.BH + kProHeads - 1) / kProHeads);
      hipLaunchKernelGGL((pool_kernel<QE, VE, D, false, true>), pgrid, dim3(256), 0, st, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL((pool_kernel<QE, VE, D, false, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PoolArgs& a, hipStream_t st) {
  if (a.qk_elt == ELT_F32) return launch_t<ELT_F32, ELT_F32, D>(a, st);
  if (a.qk_elt == ELT_BF16) return launch_t<ELT_BF16, ELT_BF16, D>(a, st);
  return launch_t<ELT_FP8, ELT_BF16, D>(a, st);
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t st) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  return a.D == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace sa
