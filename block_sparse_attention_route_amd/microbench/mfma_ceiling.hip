// Sustained bf16 MFMA rate of this device on realistic operands.
//
// The roofline of the attention kernels is quoted against MI355X's published
// dense bf16 peak.  This program measures what the matrix cores sustain when
// they do nothing else: every wave issues back-to-back
// v_mfma_f32_32x32x16_bf16 with four independent accumulators, on operands
// that are either random bf16 values (what attention sees) or one constant
// pattern.  Run it under `rocprofv3 --pmc GRBM_GUI_ACTIVE
// SQ_VALU_MFMA_BUSY_CYCLES` to see the clock and the matrix-pipe occupancy
// behind the rate.  Prints one line per variant: milliseconds and TFLOP/s.
//
//   hipcc -O3 --offload-arch=gfx950 mfma_ceiling.hip -o mfma_ceiling
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kIters = 1024;
constexpr int kThreads = 512;

template <bool RANDOM>
__global__ __launch_bounds__(kThreads, 1) void mfma_loop(float* out, const u32x4* src) {
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  bf16x8 A[8], B[8];
  for (int i = 0; i < 8; ++i) {
    if (RANDOM) {
      A[i] = __builtin_bit_cast(bf16x8, src[t * 16 + i]);
      B[i] = __builtin_bit_cast(bf16x8, src[t * 16 + 8 + i]);
    } else {
      for (int e = 0; e < 8; ++e) {
        A[i][e] = (__bf16)(1.0f + 0.001f * e);
        B[i][e] = (__bf16)(1.0f - 0.001f * e);
      }
    }
  }
  f32x16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B[i], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i + 1], B[i], a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], B[i + 1], a2, 0, 0, 0);
      a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i + 1], B[i + 1], a3, 0, 0, 0);
    }
  }
  float r = 0.f;
  for (int i = 0; i < 16; ++i) r += a0[i] + a1[i] + a2[i] + a3[i];
  out[t] = r;
}

static void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    exit(1);
  }
}

int main() {
  const int blocks = 256 * 8;
  const size_t threads = (size_t)blocks * kThreads;
  float* out = nullptr;
  u32x4* src = nullptr;
  check(hipMalloc(&out, threads * sizeof(float)), "hipMalloc out");
  check(hipMalloc(&src, threads * 16 * sizeof(u32x4)), "hipMalloc src");
  // random bf16 pairs in [-2, 2): random sign, exponent 126..127, random mantissa
  std::vector<unsigned> h(threads * 16 * 4);
  unsigned s = 12345u;
  auto next = [&]() { s = s * 1664525u + 1013904223u; return s >> 8; };
  for (auto& x : h) {
    const unsigned lo = ((next() & 1u) << 15) | ((126u + (next() & 1u)) << 7) | (next() & 127u);
    const unsigned hi = ((next() & 1u) << 15) | ((126u + (next() & 1u)) << 7) | (next() & 127u);
    x = lo | (hi << 16);
  }
  check(hipMemcpy(src, h.data(), h.size() * sizeof(unsigned), hipMemcpyHostToDevice), "hipMemcpy");
  hipEvent_t e0, e1;
  check(hipEventCreate(&e0), "event");
  check(hipEventCreate(&e1), "event");
  const double flop = (double)threads / 64 * kIters * 16 * 32768.0;
  for (int rep = 0; rep < 3; ++rep) {
    for (int m = 0; m < 2; ++m) {
      check(hipEventRecord(e0), "record");
      if (m == 0)
        hipLaunchKernelGGL(mfma_loop<true>, dim3(blocks), dim3(kThreads), 0, 0, out, src);
      else
        hipLaunchKernelGGL(mfma_loop<false>, dim3(blocks), dim3(kThreads), 0, 0, out, src);
      check(hipGetLastError(), "launch");
      check(hipEventRecord(e1), "record");
      check(hipEventSynchronize(e1), "sync");
      float ms = 0.f;
      check(hipEventElapsedTime(&ms, e0, e1), "elapsed");
      if (rep > 0)
        printf("%-18s %8.3f ms  %7.1f TFLOP/s\n", m == 0 ? "random bf16" : "constant pattern", ms,
               flop / (ms * 1e-3) / 1e12);
    }
  }
  check(hipFree(out), "free");
  check(hipFree(src), "free");
  return 0;
}
