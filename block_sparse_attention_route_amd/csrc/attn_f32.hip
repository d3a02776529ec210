// Float32 variant of the fused block-sparse attention (and of dense
// attention), for float32 Q/K/V.  Same method as the MFMA kernel -- on-chip
// routing of each query block by the shared float32 routine, the skipped
// blocks folded in as n_J copies of their mean key and value, exact attention
// over the kept blocks, one online softmax (Sol-Attn project page, section
// "Abstract") -- computed with float32 FMAs on the vector ALUs: gfx950's
// matrix cores have no full-rate float32 path, and this variant exists for
// full-precision results rather than speed.
//
// One wave per query block; lane i owns query row 64*I + i, holds q_i and its
// output accumulator in registers, and reads keys and values broadcast from
// LDS, 16 at a time, with natural exp and one rescale per group.  With the
// first-order correction a skipped block's value is its first-order value for
// this query block instead of its mean.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr int kGroup = 16;

template <int D, bool SPARSE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int N = a.N, Nb = a.Nb;
  const int bh = blockIdx.y;
  const int I = blockIdx.x;
  const int lane = threadIdx.x;

  __shared__ __attribute__((aligned(16))) float kt[kBlock * D];
  __shared__ __attribute__((aligned(16))) float vt[kBlock * D];
  __shared__ float lw[kBlock];          // log-multiplicity of each staged key
  __shared__ float p[kMaxNb];
  __shared__ uint8_t flags[SPARSE ? kMaxNb : 1];
  __shared__ float qb[D];
  __shared__ float redf[8];
  __shared__ int redi[8];
  __shared__ int counts[2];
  __shared__ int hist[SPARSE ? 256 : 1];
  __shared__ uint32_t sel[SPARSE ? 3 : 1];

  if constexpr (SPARSE) {
    for (int d = lane; d < D; d += 64) qb[d] = a.qbar[((size_t)bh * Nb + I) * D + d];
    __syncthreads();
    proxy_rows<D, 64, 1>(qb, a.kbar + (size_t)bh * Nb * D, Nb, a.scale, 1, p, (int)threadIdx.x);
    __syncthreads();
    if (a.topk > 0)
      topk_rows<64, 1>(p, Nb, 1, a.topk, flags, hist, sel, redi, counts, (int)threadIdx.x);
    else
      threshold_rows<64, 1>(p, Nb, 1, a.tau, flags, redf, redi, counts, (int)threadIdx.x);
    if (a.kept && lane == 0) a.kept[(size_t)bh * Nb + I] = counts[0];
  }

  const int row = I * kBlock + lane;   // position; its token is token_of(row)
  const bool rv = row < N;
  const size_t tok = (size_t)bh * N + (rv ? token_of(a.tm, row) : row);
  const float* qsrc = reinterpret_cast<const float*>(a.q) + tok * D;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = rv ? qsrc[d] : 0.f;
    acc[d] = 0.f;
  }
  float m = kNegInf, l = 0.f;

  // online-softmax update with `cnt` staged keys (kt, vt, lw)
  auto consume = [&](int cnt) {
    for (int g0 = 0; g0 < cnt; g0 += kGroup) {
      float x[kGroup];
      float mg = kNegInf;
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        float s = 0.f;
        if (g0 + t < cnt) {
          const float* kr = kt + (g0 + t) * D;
#pragma unroll
          for (int d = 0; d < D; ++d) s = fmaf(q[d], kr[d], s);
          x[t] = s * a.scale + lw[g0 + t];
        } else {
          x[t] = kNegInf;
        }
        mg = fmaxf(mg, x[t]);
      }
      const float mnew = fmaxf(m, mg);
      const float alpha = (m == kNegInf) ? 0.f : expf(m - mnew);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        if (g0 + t < cnt) {
          const float w = expf(x[t] - mnew);
          l += w;
          const float* vr = vt + (g0 + t) * D;
#pragma unroll
          for (int d = 0; d < D; ++d) acc[d] = fmaf(w, vr[d], acc[d]);
        }
      }
      m = mnew;
    }
  };

  const float* kin = reinterpret_cast<const float*>(a.k) + (size_t)bh * N * D;
  const float* vin = reinterpret_cast<const float*>(a.v) + (size_t)bh * N * D;

  // correction: skipped blocks as n_J copies of (kbar_J, vbar_J) -- or of
  // (kbar_J, V'[I][J]) with first-order values -- 64 at a time
  if (SPARSE && a.correction) {
    const int ntail = N - (Nb - 1) * kBlock;
    for (int J0 = 0; J0 < Nb; J0 += kBlock) {
      int cnt = 0;
      for (int J = J0; J < min(Nb, J0 + kBlock); ++J) {
        if (flags[J] & 1) continue;
        const float* kb = a.kbar + ((size_t)bh * Nb + J) * D;
        const float* vb = a.vprime32 ? a.vprime32 + (((size_t)bh * Nb + I) * Nb + J) * D
                                     : a.vbar + ((size_t)bh * Nb + J) * D;
        for (int d = lane; d < D; d += 64) {
          kt[cnt * D + d] = kb[d];
          vt[cnt * D + d] = vb[d];
        }
        if (lane == 0) lw[cnt] = logf((float)(J == Nb - 1 ? ntail : kBlock));
        ++cnt;
      }
      __syncthreads();
      consume(cnt);
      __syncthreads();
    }
  }

  // exact attention over the kept blocks (all blocks when dense)
  for (int J = 0; J < Nb; ++J) {
    if (SPARSE && !(flags[J] & 1)) continue;
    const int n = min(kBlock, N - J * kBlock);
    if (a.tm.on) {
      for (int r = 0; r < n; ++r) {
        const size_t t = (size_t)token_of(a.tm, J * kBlock + r) * D;
        for (int d = lane; d < D; d += 64) {
          kt[r * D + d] = kin[t + d];
          vt[r * D + d] = vin[t + d];
        }
      }
    } else {
      for (int x = lane; x < n * D; x += 64) {
        kt[x] = kin[(size_t)J * kBlock * D + x];
        vt[x] = vin[(size_t)J * kBlock * D + x];
      }
    }
    if (lane < n) lw[lane] = 0.f;
    __syncthreads();
    consume(n);
    __syncthreads();
  }

  if (rv) {
    const float inv = 1.f / l;
    float* orow = reinterpret_cast<float*>(a.o) + tok * D;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
    a.lse[tok] = m + logf(l);
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.Nb, a.BH);
  if (a.sparse)
    hipLaunchKernelGGL((attn_f32_kernel<D, true>), grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_f32_kernel<D, false>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  return a.D == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace sa
