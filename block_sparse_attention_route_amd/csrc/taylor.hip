// First-order values of the skipped blocks (correction mode 2) for gfx950.
//
// Paper review of the Sol Video Inference Engine (xllm-io blog, five
// acceleration techniques, item "Sparse Attention"): PISA computes the
// critical blocks exactly and compensates the others with a first-order
// Taylor approximation.  Expanding the weight exp(s q_i . k_j) of a key of a
// skipped block J to first order in the key's deviation d_j = k_j - kbar_J,
// with the coefficient taken at the query block mean qbar_I (the product of
// the query's and the key's deviations is second order and dropped), leaves
// the block's weight n_J exp(s q_i . kbar_J) as it is and replaces its value
// by
//
//   V'[I][J] = vbar_J + (s / n_J) * sum_{j in J} (qbar_I . d_j) v_j,
//
// one D-vector per (query block, key block).  This kernel writes all of them,
// bf16, [BH][Nb][Nbp][D], rows J >= Nb zero; the fused attention kernel then
// reads rows [I][64c, 64c + 64) as the values of correction tile c.
//
// Workgroup: one head, 256 query blocks (eight waves of 32, one per lane
// column) and one chunk of 64 key blocks.  With c = s / 64 and qc_I =
// bf16(c qbar_I), for each key block J it computes, like an attention tile
// with the scaled block means as queries,
//   S~^T = K_J qc^T - r_IJ  v_mfma_f32_32x32x16_bf16, the accumulator starting
//                           at -r_IJ = -qc_I . kbar_J (kbar_J split into two
//                           bf16 halves, v_dot2_f32_bf16): centred scores,
//                           whose sum over the block vanishes; keys past the
//                           end of the sequence give 0, and the ragged last
//                           block scales them by 64 / n_J
//   V'^T = vbar_J + V_J^T bf16(S~^T)   the same MFMA, the accumulator starting
//                           at vbar_J, V_J^T from the regrouped V
// and writes V' in bf16.  The K and V^T tiles of the next key block are
// fetched into registers while the current one is used and handed over
// through a second LDS buffer, so one barrier per key block suffices.  With
// fp8 K the codes are widened to bf16 (exactly) on their way into LDS and the
// block scale multiplies the score accumulator (S~ = scale_J * (codes . qc) -
// r_IJ, the block mean kbar_J being that of the dequantised keys).  Each
// wave turns its 32 output rows around in LDS and writes them as whole rows,
// 16 bytes per lane (written straight from the MFMA layout, every store
// would touch 32 rows).
#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {
namespace {

constexpr int kTyWaves = 8;             // waves per workgroup
constexpr int kTyRows = 32 * kTyWaves;  // query blocks per workgroup
constexpr int kTyThreads = 64 * kTyWaves;

template <int D>
struct TyCfg {
  static constexpr int KS = D / 16;           // k-steps of S^T
  static constexpr int DT = D / 32;           // 32-row d tiles of U^T
  static constexpr int KROW = 2 * D;          // bytes of a bf16 K row
  static constexpr int CPR = KROW / 16;       // 16-byte chunks per K row
  static constexpr int KTILE = 64 * KROW;     // K tile: 64 keys
  static constexpr int VTILE = D * 128;       // V^T tile: D rows of 64 bf16 keys
  static constexpr int KLD = KTILE / 16 / kTyThreads;  // 16-byte copies per thread
  static constexpr int VLD = VTILE / 16 / kTyThreads;
  static constexpr int OST = 32 * KROW / 16 / 64;   // 16-byte output stores per lane: 32 rows of D bf16
  static constexpr int K8C = 64 * D / 16;             // 16-byte chunks of an fp8 K tile
  static constexpr int KLD8 = (K8C + kTyThreads - 1) / kTyThreads;
};

template <int D, bool K8>
__global__ __launch_bounds__(kTyThreads, 1) void taylor_kernel(TaylorArgs a) {
  using C = TyCfg<D>;
  static_assert(C::KLD >= 1 && C::VLD >= 1, "tile copies per thread");
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][C::KTILE];
  __shared__ __attribute__((aligned(16))) uint8_t vt[2][C::VTILE];
  __shared__ __attribute__((aligned(16))) __bf16 kbh[2][2][D];   // kbar_J: bf16 high and low parts
  __shared__ __attribute__((aligned(16))) float vb[2][D];
  // per wave: its 32 output rows of the current key block, 16-byte chunks
  // XOR-swizzled by row, so that the rows go out as whole rows
  __shared__ __attribute__((aligned(16))) uint8_t ost[kTyWaves][32 * C::KROW];

  const int N = a.N, Nb = a.Nb, Nbp = a.Nbp;
  const int nit = (Nb + kTyRows - 1) / kTyRows;
  const int nch = Nbp / 64;
  const int G = a.BH * nch * nit;
  const int t = xcd_remap<16>((int)blockIdx.x, G);
  const int bh = t / (nch * nit);
  const int rem = t - bh * (nch * nit);
  const int ch = rem / nit, itile = rem - ch * nit;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, l32 = lane & 31;
  const int I = kTyRows * itile + 32 * wave + l32;   // this lane's query block
  const bool ivalid = I < Nb;
  const int J0 = 64 * ch;
  const int Jend = min(J0 + 64, Nb);                  // key blocks with data
  const int ntail = N - (Nb - 1) * kBlock;

  // qc_I = bf16(s / 64 * qbar_I): the B operand of S~^T
  const float c64 = a.scale / (float)kBlock;
  bf16x8 qr[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    bf16x8 x = {};
    if (ivalid) {
      const float* src = a.qbar + ((size_t)bh * Nb + I) * D + 16 * ks + 8 * h;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = static_cast<__bf16>(c64 * lo[e]);
        x[e + 4] = static_cast<__bf16>(c64 * hi[e]);
      }
    }
    qr[ks] = x;
  }

  // Copies of key block J: per thread KLD + VLD 16-byte chunks of the K and
  // V^T tiles, and one of the kbar / vbar rows for the first D/2 threads.
  u32x4 kr[K8 ? C::KLD8 : C::KLD], vr[C::VLD], mr;
  auto fetch = [&](int J) {
    const int nJ = (J == Nb - 1) ? ntail : kBlock;
    if constexpr (K8) {
      // fp8 codes, 16 per chunk, in row order (the swizzle is applied when stored)
      const uint8_t* kbase = a.k8 + ((size_t)bh * N + (size_t)J * kBlock) * D;
#pragma unroll
      for (int i = 0; i < C::KLD8; ++i) {
        const int P = tid + kTyThreads * i, row = P / (D / 16), pc = P % (D / 16);
        if (P < C::K8C)
          kr[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)min(row, nJ - 1) * D + pc * 16);
      }
    } else {
      const uint16_t* kbase = a.k + ((size_t)bh * N + (size_t)J * kBlock) * D;
#pragma unroll
      for (int i = 0; i < C::KLD; ++i) {
        const int P = tid + kTyThreads * i, row = P / C::CPR, pc = P % C::CPR;
        const int src_row = min(row, nJ - 1);   // rows past the sequence end: finite data, zeroed later
        kr[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)src_row * D + swz<C::CPR>(row, pc) * 8);
      }
    }
    const uint16_t* vbase = a.vt16 + ((size_t)bh * Nb + J) * D * kBlock;
#pragma unroll
    for (int i = 0; i < C::VLD; ++i) {
      const int P = tid + kTyThreads * i, row = P / 8, pc = P % 8;
      vr[i] = *reinterpret_cast<const u32x4*>(vbase + row * 64 + swz<8>(row, pc) * 8);
    }
    if (tid < D / 2) {
      const float* m = (tid < D / 4 ? a.kbar : a.vbar) + ((size_t)bh * Nb + J) * D + 4 * (tid % (D / 4));
      mr = *reinterpret_cast<const u32x4*>(m);
    }
  };
  auto stash = [&](int buf) {
    if constexpr (K8) {
#pragma unroll
      for (int i = 0; i < C::KLD8; ++i) {
        const int P = tid + kTyThreads * i, row = P / (D / 16), pc = P % (D / 16);
        if (P < C::K8C) {
          // 16 codes -> two bf16 chunks (exact), logical chunks 2 pc and 2 pc + 1
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            bf16x8 x;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              x[e] = static_cast<__bf16>(fp8e4m3_to_f32((kr[i][2 * half + (e >> 2)] >> (8 * (e & 3))) & 0xFFu));
            *reinterpret_cast<bf16x8*>(&kt[buf][row * C::KROW + swz<C::CPR>(row, 2 * pc + half) * 16]) = x;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::KLD; ++i) {
        const int P = tid + kTyThreads * i;
        *reinterpret_cast<u32x4*>(&kt[buf][16 * P]) = kr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::VLD; ++i) {
      const int P = tid + kTyThreads * i;
      *reinterpret_cast<u32x4*>(&vt[buf][16 * P]) = vr[i];
    }
    if (tid < D / 4) {
      // kbar = hi + lo with both parts in bf16 (relative error 2^-16)
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __uint_as_float(mr[e]);
        hi[e] = static_cast<__bf16>(x);
        lo[e] = static_cast<__bf16>(x - static_cast<float>(hi[e]));
      }
      *reinterpret_cast<bf16x4*>(&kbh[buf][0][4 * tid]) = hi;
      *reinterpret_cast<bf16x4*>(&kbh[buf][1][4 * tid]) = lo;
    } else if (tid < D / 2) {
      *reinterpret_cast<u32x4*>(&vb[buf][4 * (tid - D / 4)]) = mr;
    }
  };

  if (J0 < Jend) {
    fetch(J0);
    stash(0);
  }
  __syncthreads();

  for (int j = 0; j < 64; ++j) {
    const int J = J0 + j, buf = j & 1;
    const bool more = J + 1 < Jend;
    if (more) fetch(J + 1);
    // output rows of this wave: 16 bytes per lane and store, whole rows
    auto store_rows = [&](auto chunk_of) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < C::OST; ++i) {
        const int q = 64 * i + lane, row = q / C::CPR, c = q % C::CPR;
        const int Ir = kTyRows * itile + 32 * wave + row;
        const u32x4 x = chunk_of(row, c);
        if (Ir < Nb)
          *reinterpret_cast<u32x4*>(a.vprime + (((size_t)bh * Nb + Ir) * Nbp + J) * D + 8 * c) = x;
      }
    };
    if (J < Jend) {
      const uint8_t* Kb = kt[buf];
      const uint8_t* Vb = vt[buf];
      // r_IJ = qc_I . kbar_J: this lane's half of d, plus lane^32's
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      float rp = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 kh = *reinterpret_cast<const bf16x8*>(&kbh[buf][0][16 * ks + 8 * h]);
        const bf16x8 kl = *reinterpret_cast<const bf16x8*>(&kbh[buf][1][16 * ks + 8 * h]);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 qp = {qr[ks][e], qr[ks][e + 1]};
          const bf16x2 hp = {kh[e], kh[e + 1]};
          const bf16x2 lp = {kl[e], kl[e + 1]};
          rp = __builtin_amdgcn_fdot2_f32_bf16(qp, hp, rp, false);
          rp = __builtin_amdgcn_fdot2_f32_bf16(qp, lp, rp, false);
        }
      }
      const float r = rp + __shfl_xor(rp, 32);

      // S~^T = K_J qc^T - r_IJ (fp8: scale_J * (codes qc^T) - r_IJ, below)
      float sk = 1.f;
      if constexpr (K8) sk = a.k_scale[(size_t)bh * Nb + J];
      f32x16 sc[2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[k2][e] = K8 ? 0.f : -r;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int krow = 32 * k2 + kperm(l32);
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Kb + krow * C::KROW + swz<C::CPR>(krow, 2 * ks + h) * 16);
          sc[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qr[ks], sc[k2], 0, 0, 0);
        }
      }
      // centred scores in bf16, the B operand of V'^T; the ragged last block:
      // keys past the sequence end give 0, the others are scaled to s / n_J
      bf16x8 pb[4];
      if (J == Nb - 1 && ntail < kBlock) {
        const float f = (float)kBlock / (float)ntail;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const bool live = 32 * k2 + key_of(e, h) < ntail;
            const float x = K8 ? fmaf(sk, sc[k2][e], -r) : sc[k2][e];
            pb[2 * k2 + (e >> 3)][e & 7] = static_cast<__bf16>(live ? x * f : 0.f);
          }
      } else {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            pb[2 * k2 + (e >> 3)][e & 7] = static_cast<__bf16>(K8 ? fmaf(sk, sc[k2][e], -r) : sc[k2][e]);
      }

      // V'^T = vbar_J + V_J^T S~^T
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const int vrow = 32 * dt + l32;
        f32x16 acc;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 vm = *reinterpret_cast<const f32x4*>(&vb[buf][32 * dt + 8 * g + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * g + e] = vm[e];
        }
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vb + vrow * 128 + swz<8>(vrow, 2 * k4 + h) * 16);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[k4], acc, 0, 0, 0);
        }
        // row l32 of the wave's staging area, d = 32 dt + 8 g + 4 h .. + 3
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = (uint32_t)f32_to_bf16_bits(acc[4 * g + 0]) | ((uint32_t)f32_to_bf16_bits(acc[4 * g + 1]) << 16);
          w[1] = (uint32_t)f32_to_bf16_bits(acc[4 * g + 2]) | ((uint32_t)f32_to_bf16_bits(acc[4 * g + 3]) << 16);
          const int c = 4 * dt + g;
          *reinterpret_cast<u32x2*>(&ost[wave][l32 * C::KROW + (c ^ (l32 & (C::CPR - 1))) * 16 + 8 * h]) = w;
        }
      }
      // the wave's own staging area: no barrier, LDS accesses of a wave are ordered
      store_rows([&](int row, int c) {
        return *reinterpret_cast<const u32x4*>(&ost[wave][row * C::KROW + (c ^ (row & (C::CPR - 1))) * 16]);
      });
    } else {
      // key blocks J >= Nb: zero rows (the attention kernel masks them, but
      // reads them as MFMA operands)
      store_rows([](int, int) { return u32x4{0u, 0u, 0u, 0u}; });
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
  }
}

// Float32 values for the float32 path (correctness rather than speed): one
// wave per (query block, head); per key block J, lane j forms the centred
// score qbar_I . (k_j - kbar_J) of key j, then lane d sums the keys' values
// in column d.  Rows are read through the position -> token map.  Only
// J < Nb is written ([BH][Nb][Nb][D]).
template <int D>
__global__ __launch_bounds__(64) void taylor_f32_kernel(TaylorArgs a) {
  const int N = a.N, Nb = a.Nb;
  const int bh = blockIdx.y, I = blockIdx.x, lane = threadIdx.x;
  __shared__ float qb[D];
  __shared__ float t[kBlock];
  __shared__ int tok[kBlock];
  for (int d = lane; d < D; d += 64) qb[d] = a.qbar[((size_t)bh * Nb + I) * D + d];
  const float* kin = a.kf + (size_t)bh * N * D;
  const float* vin = a.vf + (size_t)bh * N * D;
  const int ntail = N - (Nb - 1) * kBlock;
  for (int J = 0; J < Nb; ++J) {
    const int n = (J == Nb - 1) ? ntail : kBlock;
    tok[lane] = lane < n ? token_of(a.tm, J * kBlock + lane) : 0;
    __syncthreads();
    const float* kb = a.kbar + ((size_t)bh * Nb + J) * D;
    float tj = 0.f;
    if (lane < n) {
      const float* kr = kin + (size_t)tok[lane] * D;
      for (int d = 0; d < D; ++d) tj = fmaf(qb[d], kr[d] - kb[d], tj);
    }
    t[lane] = tj;
    __syncthreads();
    const float c = a.scale / (float)n;
    const float* vb = a.vbar + ((size_t)bh * Nb + J) * D;
    float* out = a.vprime32 + (((size_t)bh * Nb + I) * Nb + J) * D;
    for (int d = lane; d < D; d += 64) {
      float u = 0.f;
      for (int j = 0; j < n; ++j) u = fmaf(t[j], vin[(size_t)tok[j] * D + d], u);
      out[d] = fmaf(c, u, vb[d]);
    }
    __syncthreads();
  }
}

template <int D>
hipError_t launch_f32(const TaylorArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(taylor_f32_kernel<D>, dim3(a.Nb, a.BH), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const TaylorArgs& a, hipStream_t st) {
  const int nit = (a.Nb + kTyRows - 1) / kTyRows;
  const dim3 grid((unsigned)(a.BH * (a.Nbp / 64) * nit));
  if (a.k8)
    hipLaunchKernelGGL((taylor_kernel<D, true>), grid, dim3(kTyThreads), 0, st, a);
  else
    hipLaunchKernelGGL((taylor_kernel<D, false>), grid, dim3(kTyThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_taylor(const TaylorArgs& a, hipStream_t st) {
  if (a.BH == 0 || a.Nb == 0) return hipSuccess;
  if (a.vprime32) return a.D == 64 ? launch_f32<64>(a, st) : launch_f32<128>(a, st);
  return a.D == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace sa
