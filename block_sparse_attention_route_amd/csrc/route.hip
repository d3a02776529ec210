// Step "route", standalone (the fused attention kernel runs the same device
// routine on chip and never writes a mask): for each query block I of each
// head, p_IJ = s * qbar_I . kbar_J over all key blocks J, its row maximum,
// and the 0/1 keep mask p_IJ >= max_J p_IJ - tau (Sol-Attn project page,
// section "Abstract": query-dependent threshold routing on a pooled score),
// or, with a fixed budget topk > 0, the topk largest p_IJ of the row (PISA's
// fixed sparsity in the paper review of the Sol Video Inference Engine).
//
// One workgroup routes two adjacent query blocks of one head, exactly as the
// fused kernel does, so that both obtain the same float32 bits.
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  const int pair = blockIdx.x;
  const int bh = blockIdx.y;
  const int I0 = 2 * pair;
  const bool two = I0 + 1 < a.Nb;

  __shared__ float qb[2 * D];
  __shared__ float p[2 * kMaxNb];
  __shared__ uint8_t flags[kMaxNb];
  __shared__ float redf[8];
  __shared__ int redi[8];
  __shared__ int counts[2];
  __shared__ int hist[2 * 256];
  __shared__ uint32_t sel[6];

  const int tid = threadIdx.x;
  if (tid < 2 * D) {
    const int r = tid / D, d = tid % D;
    const int I = I0 + r;
    qb[tid] = (I < a.Nb) ? a.qbar[((size_t)bh * a.Nb + I) * D + d] : 0.f;
  }
  __syncthreads();
  proxy_rows<D, 256, 2>(qb, a.kbar + (size_t)bh * a.Nb * D, a.Nb, a.scale, two ? 2 : 1, p, tid);
  __syncthreads();
  if (a.topk > 0)
    topk_rows<256, 2>(p, a.Nb, two ? 2 : 1, a.topk, flags, hist, sel, redi, counts, tid);
  else
    threshold_rows<256, 2>(p, a.Nb, two ? 2 : 1, a.tau, flags, redf, redi, counts, tid);

  uint8_t* m0 = a.mask + ((size_t)bh * a.Nb + I0) * a.Nb;
  for (int J = tid; J < a.Nb; J += 256) {
    const uint8_t f = flags[J];
    m0[J] = f & 1;
    if (two) m0[a.Nb + J] = (f >> 1) & 1;
  }
  if (a.kept && tid == 0) {
    a.kept[(size_t)bh * a.Nb + I0] = counts[0];
    if (two) a.kept[(size_t)bh * a.Nb + I0 + 1] = counts[1];
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.BH == 0 || a.Nb == 0) return hipSuccess;
  dim3 grid((a.Nb + 1) / 2, a.BH);
  if (a.D == 64)
    hipLaunchKernelGGL(route_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(route_kernel<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sa
