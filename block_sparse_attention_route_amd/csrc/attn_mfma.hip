// Fused on-the-fly block-sparse flash attention for gfx950 (bf16 MFMA; fp8
// QK^T variant), and the dense attention it reduces to.
//
// Sol-Attn project page (section "Abstract"): routing by a query-dependent
// threshold, sparse computation and an approximate correction of the skipped
// blocks run in a single online-softmax pass, with blocks selected on chip and
// no proxy map materialised.  Sol-Engine README (section "Sol-Attention"):
// only the most relevant key blocks are computed, plus a light-weight
// compensating operation.  Per workgroup (QB adjacent 64-token query blocks
// of one head) this kernel:
//
//   1. route: evaluates the proxy rows p_IJ = s * qbar_I . kbar_J of its
//      query blocks into LDS (the shared float32 routine of sa_device.h),
//      thresholds them at rowmax - tau (or keeps each row's topk largest,
//      the fixed-budget mode) and compacts the union of the kept key blocks
//      into an index list in LDS -- nothing is written to HBM;
//   2. correct: streams the block means as "virtual keys": virtual key J has
//      key kbar_J, value vbar_J and log-multiplicity log(n_J), and is masked
//      for a query block that keeps J.  Its logit s * q_i . kbar_J is entry
//      (i, J) of s * Q_I Kbar^T -- the below-threshold score column of block
//      J -- and it enters the same running max / sum as the exact keys.  With
//      the first-order correction (TAY; the paper review of the Sol Video
//      Inference Engine, xllm-io blog, five acceleration techniques, item
//      "Sparse Attention": non-critical blocks compensated to first order)
//      the value of virtual key J is its first-order value for this query
//      block, V'[I][J] from the workspace, staged per query block in LDS;
//   3. exact: flash attention over the kept key blocks (the union list; the
//      waves of a query block that does not keep a block skip it), with the
//      ragged last key block masked;
//   4. epilogue: O = acc / l in bf16 and the natural-log LSE.
//
// Tiling.  A workgroup takes QB adjacent query blocks (QB = 4 at D = 128, 2
// at D = 64) with two waves per block; wave w owns 32 query rows (query block
// QB*group + w/2, rows 32*(w%2) ..) against the full 64-key tile.  Products
// use v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x64_f8f6f4 for fp8 Q K^T)
// with the roles transposed, S^T = K Q^T and O^T = V^T P^T: a lane owns one
// query column, so the softmax row max and sum are lane-local plus one
// exchange with lane^32, and the exponentiated scores are already the B
// operand of the PV product.  The MFMA row order of K is permuted (bits 2 and
// 3 swapped) so that the keys a lane holds after S^T are exactly the keys its
// PV operand needs.  K tiles are row-major and V tiles arrive pre-transposed
// (d-major) from the pool step; both are copied straight from global memory
// into a ring of LDS stages (LDS DMA, global_load_lds_dwordx4) issued one
// tile ahead, from a wave-uniform base address plus per-lane offsets computed
// once, with an XOR swizzle on 16-byte chunks that keeps the MFMA operand
// reads free of bank conflicts; the tile loop is unrolled by ring stage so
// that the LDS operand addresses are immediates.  Work is ordered so that
// each XCD takes chunks of adjacent query blocks while all XCDs stay on the
// same head (shared key blocks hit in that XCD's L2, the head's K/V stays in
// the last-level cache): the dense kernel remaps its workgroup ids; the
// sparse kernel, whose groups differ in cost, runs one persistent workgroup
// per CU that takes groups from its XCD's queue and, once that is empty,
// from the other XCDs' queues.
//
// Softmax.  The running maximum is raised lazily and without a per-tile
// maximum: the weights P = 2^(s - m) are taken against the maximum in use,
// and only when some row's weights of a tile exceed 2^64 (or overflow) are
// the row maxima taken, l and the accumulators rescaled and the tile's
// weights redone.  This is exact -- numerator and denominator carry the same
// stale maximum, and weights up to 2^64 keep their relative precision in
// bf16 and fp32 -- and makes the rescale rare (in practice a row's first
// tile).  Row sums are taken over the bf16-rounded P that enters the PV
// product.
#include <algorithm>
#include <type_traits>

#include "sa_device.h"
#include "sa_kernels.h"

namespace sa {
namespace {

// The running maximum is raised lazily: weights are taken against it as it
// stands, and only a tile whose weights exceed kWeightMax (2^64) raises it.
constexpr float kWeightMax = 18446744073709551616.0f;
constexpr float kMInit = -1e30f;  // finite start of the running maximum

// Kinds of key tile: block means (correction), a full exact block, the
// ragged last exact block.
constexpr int kVirt = 0, kPlain = 1, kTail = 2;

// max of x over lanes l and l^32 (v_permlane32_swap exchanges the halves)
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int CPR>
__device__ __forceinline__ int swz_any(int row, int chunk) {
  if constexpr (CPR == 4) {
    return chunk ^ ((row >> 2) & 3);
  } else {
    return swz<CPR>(row, chunk);
  }
}

template <int NT>
__device__ __forceinline__ void build_union(const uint8_t* __restrict__ flags, int Nb,
                                            uint16_t* __restrict__ ulist, int* total, int* wsum, int tid) {
  constexpr int NW = NT / 64;
  const int lane = tid & 63, wave = tid >> 6;
  const int seg = (Nb + NT - 1) / NT;
  const int j0 = min(Nb, tid * seg), j1 = min(Nb, j0 + seg);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += flags[j] != 0;
  int x = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) base += (w < wave) ? wsum[w] : 0;
  int pos = base + x - cnt;
  for (int j = j0; j < j1; ++j) {
    const int f = flags[j];
    if (f) ulist[pos++] = (uint16_t)(j | (f << 12));
  }
  if (tid == NT - 1) *total = base + x;
  __syncthreads();
}

template <int D>
struct Cfg {
  static constexpr int KS = D / 16;          // k-steps of S^T (bf16 K)
  static constexpr int DT = D / 32;          // 32-row d tiles of O^T
  static constexpr int KROW16 = 2 * D;       // bytes of a bf16 K row
  static constexpr int CPR16 = KROW16 / 16;  // 16-byte chunks per bf16 K row
  static constexpr int KROW8 = D;            // bytes of an fp8 K row
  static constexpr int CPR8 = KROW8 / 16;
  static constexpr int KTILE = 64 * KROW16;  // K buffer bytes (sized for bf16)
  static constexpr int VTILE = D * 128;      // V^T tile: D rows of 64 bf16 keys
};

// 16 bytes per lane from global memory straight into LDS (LDS DMA): lane l's
// bytes land at lds_wave_base + 16*l.  Issued as inline assembly so that the
// compiler does not order every later LDS read behind the copy; the kernel
// waits for each tile itself (vmcnt) before the barrier that publishes it.
// The copy takes its LDS address from M0, which the compiler owns: the
// statement saves M0 and restores it, so M0 is unchanged across it.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_wave_base))
               : "memory");
}

// The same copy from a wave-uniform base address (scalar registers) plus a
// per-lane 32-bit byte offset, so a tile's copies need no per-lane address
// arithmetic once the offsets are known.
__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ void dma16s(uint32_t voff, uint64_t sbase, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_wave_base))
               : "memory");
}

// One float from a wave-uniform global address through the scalar unit,
// waited for inside the same statement: a vector load here would make the
// compiler wait for the in-flight tile copies as well.
__device__ __forceinline__ float scalar_load_f32(const float* p) {
  float v;
  // readfirstlane is a 32-bit operation: make each half of the address uniform
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  const uint64_t up = ((uint64_t)hi << 32) | lo;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(up) : "memory");
  return v;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int LPT, int MAXAHEAD>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  // all but the last ahead*LPT vector-memory loads of this thread complete
  if constexpr (MAXAHEAD >= 3) {
    if (ahead >= 3) { wait_vmcnt<3 * LPT>(); return; }
  }
  if constexpr (MAXAHEAD >= 2) {
    if (ahead == 2) { wait_vmcnt<2 * LPT>(); return; }
  }
  if constexpr (MAXAHEAD >= 1) {
    if (ahead == 1) { wait_vmcnt<LPT>(); return; }
  }
  wait_vmcnt<0>();
}

// Group i of XCD x's queue under the XCD-aware order xcd_remap<CH> (the
// groups that order places on XCD x, in the same order), or -1 past its end.
template <int CH>
__device__ __forceinline__ int xcd_queue_group(int x, int i, int G) {
  const int rounds = G / (8 * CH);
  if (i < rounds * CH) return (i / CH) * (8 * CH) + x * CH + (i % CH);
  const int g = rounds * 8 * CH + 8 * (i - rounds * CH) + x;
  return g < G ? g : -1;
}

// Next group for a persistent workgroup on XCD x: its own XCD's queue first,
// then the other queues in turn; -1 once every queue is empty.  sched[0..7]
// count the groups taken from each queue (zeroed before the launch).
template <int CH>
__device__ __forceinline__ int grab_group(int* sched, int x, int G) {
#pragma unroll 1
  for (int t = 0; t < 8; ++t) {
    const int y = (x + t) & 7;
    // skip a queue seen empty without taking a ticket from it
    if (xcd_queue_group<CH>(y, __hip_atomic_load(&sched[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), G) < 0)
      continue;
    const int g = xcd_queue_group<CH>(y, atomicAdd(&sched[y], 1), G);
    if (g >= 0) return g;
  }
  return -1;
}

__global__ void reset_sched(int* sched) {
  if (threadIdx.x < 8) sched[threadIdx.x] = 0;
}

template <int D, bool SPARSE, bool FP8, int QB, int ST, bool TAY = false>
__global__ __launch_bounds__(128 * QB, QB == 2 ? 2 : 1) void attn_kernel(AttnArgs a) {
  using C = Cfg<D>;
  constexpr int NT = 128 * QB;        // threads
  constexpr int NW = 2 * QB;          // waves: two 32-row halves per query block
  constexpr int KI16 = C::KTILE / 1024 / NW;       // per-thread DMA copies, bf16 K tile
  constexpr int KI8 = C::KTILE / 2 / 1024 / NW;    // fp8 K tile
  constexpr int VI = C::VTILE / 1024 / NW;         // V^T tile
  constexpr int LPT = (FP8 ? (KI8 < KI16 ? KI8 : KI16) : KI16) + VI;  // fewest copies per tile
  // A ring stage holds a K tile and a V^T tile.  Correction tiles take the
  // key means in two bf16 halves: the low half goes to a third buffer of the
  // stage, or, with first-order values (whose PV operand comes from its own
  // LDS area), to the V^T buffer.
  constexpr int STAGE = C::KTILE + C::VTILE + ((SPARSE && !TAY) ? C::KTILE : 0);
  constexpr int LO_OFF = TAY ? C::KTILE : C::KTILE + C::VTILE;
  constexpr int SMEM_STAGE = ST * STAGE;
  // The routing step's arrays (proxies, per-block flags, the fixed-budget
  // histograms, the query means) are dead once the union list is built, and
  // share the ring's LDS: the first tile is issued after that.
  constexpr int R_FLAGS = QB * kMaxNb * 4, R_HIST = R_FLAGS + kMaxNb, R_QB = R_HIST + QB * 256 * 4;
  constexpr int SMEM_ROUTE = SPARSE ? R_QB + QB * D * 4 : 0;
  constexpr int SMEM = SMEM_STAGE > SMEM_ROUTE ? SMEM_STAGE : SMEM_ROUTE;
  static_assert(KI8 >= 1 && VI >= 1, "tile copies per wave");
  static_assert(!TAY || SPARSE, "first-order values: sparse only");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
  uint8_t* const flags = smem + R_FLAGS;
  int* const hist = reinterpret_cast<int*>(smem + R_HIST);
  float* const qb = reinterpret_cast<float*>(smem + R_QB);
  __shared__ uint16_t ulist[SPARSE ? kMaxNb : 1];
  __shared__ uint64_t skipbits[SPARSE ? QB * (kMaxNb / 64) : 1];  // per query block, per 64-block chunk
  __shared__ float redf[QB * NW];
  __shared__ int redi[QB * NW];
  __shared__ int counts[QB];
  __shared__ uint32_t sel[SPARSE ? 3 * QB : 1];
  __shared__ int nunion_s;
  // correction mode 2: the first-order value tile of each query block, 64 key
  // rows of D bf16, unswizzled (operands are gathered from it per element)
  __shared__ __attribute__((aligned(16))) uint8_t vps[TAY ? QB * C::KTILE : 1];

  __shared__ int next_tile_s;

  const int G = a.BH * ((a.Nb + QB - 1) / QB);
  // Dense: one group per workgroup, XCD-aware order.  Sparse: groups differ
  // in cost, so a persistent grid takes them from the per-XCD queues (each
  // XCD's queue holds the groups the XCD-aware order gives it) and, once its
  // own queue is empty, from the other XCDs' queues.
  int tile_next = SPARSE ? -1 : xcd_remap<SA_XCD_CHUNK>((int)blockIdx.x, G);
  for (;;) {
  if constexpr (SPARSE) {
    if (threadIdx.x == 0) next_tile_s = grab_group<SA_XCD_CHUNK_SPARSE>(a.sched, (int)blockIdx.x & 7, G);
    __syncthreads();
    tile_next = next_tile_s;
  }
  const int tile = tile_next;
  if (tile < 0) break;
  // The thread index and the sizes pass through empty asm statements, so
  // that nothing derived from them is hoisted out of the group loop: kept
  // live across every group, those values would crowd the registers of the
  // tile loop.
  int tid_opaque = threadIdx.x, N_opaque = a.N, Nb_opaque = a.Nb;
  asm volatile("" : "+v"(tid_opaque), "+s"(N_opaque), "+s"(Nb_opaque));
  const int N = N_opaque, Nb = Nb_opaque;
  const int ngroups = (Nb + QB - 1) / QB;
  const int bh = tile / ngroups;
  const int grp = tile - bh * ngroups;
  const int tid = tid_opaque, wave = tid >> 6, lane = tid & 63;
  const int qsel = wave >> 1, qhalf = wave & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int I = QB * grp + qsel;
  const bool qvalid = I < Nb;
  const int nrows = min(QB, Nb - QB * grp);   // valid query blocks of this group
  const int ntail = N - (Nb - 1) * kBlock;    // tokens in the last block
  const int nchunks = (Nb + 63) >> 6;          // 64-block chunks of virtual keys

  // ---------------------------------------------------------------- 1. route
  int nvirt = 0, nunion = Nb;
  if constexpr (SPARSE) {
    for (int t = tid; t < QB * D; t += NT) {
      const int r = t / D, d = t % D;
      qb[t] = (r < nrows) ? a.qbar[((size_t)bh * Nb + QB * grp + r) * D + d] : 0.f;
    }
    __syncthreads();
    float* p = reinterpret_cast<float*>(smem);
    proxy_rows<D, NT, QB>(qb, a.kbar + (size_t)bh * Nb * D, Nb, a.scale, nrows, p, tid);
    __syncthreads();
    if (a.topk > 0)
      topk_rows<NT, QB>(p, Nb, nrows, a.topk, flags, hist, sel, redi, counts, tid);
    else
      threshold_rows<NT, QB>(p, Nb, nrows, a.tau, flags, redf, redi, counts, tid);
    build_union<NT>(flags, Nb, ulist, &nunion_s, redi, tid);
    nunion = nunion_s;
    if (a.kept && tid < nrows) a.kept[(size_t)bh * Nb + QB * grp + tid] = counts[tid];
    if (a.correction) {
      nvirt = nchunks;
      // skipbits[r][c] bit j: block 64c + j exists and query block r skips it
      for (int rc = wave; rc < QB * nchunks; rc += NW) {
        const int r = rc / nchunks, c = rc - r * nchunks;
        const int J = 64 * c + lane;
        const bool skip = J < Nb && !((flags[J < Nb ? J : 0] >> r) & 1);
        const uint64_t bits = __ballot(skip);
        if (lane == 0) skipbits[r * (kMaxNb / 64) + c] = bits;
      }
      __syncthreads();
    }
  }
  const int ntiles = nvirt + nunion;

  // --------------------------------------- query operands (B of S^T = K Q^T)
  const int qrow = I * kBlock + 32 * qhalf + l32;  // this lane's query row
  const bool rowvalid = qvalid && qrow < N;
  // position qrow holds token token_of(qrow): the raster order, or the 3-D tile order
  const size_t qtok = (size_t)bh * N + (rowvalid ? token_of(a.tm, qrow) : qrow);
  bf16x8 qr[C::KS];
  // fp8 Q codes as the B operand of v_mfma_f32_32x32x64_f8f6f4: product m
  // contracts dims [64m, 64m + 64); lane half h holds the 32 codes of dims
  // [64m + 32h, 64m + 32h + 32), the same dims its K operand holds
  i32x8 q8[FP8 ? D / 64 : 1];
  if constexpr (FP8) {
    const uint8_t* qrow8 = reinterpret_cast<const uint8_t*>(a.q) + qtok * D;
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      i32x8 w = {};
      if (rowvalid) w = *reinterpret_cast<const i32x8*>(qrow8 + 64 * m + 32 * h);
      q8[m] = w;
    }
  }
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const int d0 = 16 * ks + 8 * h;
    if constexpr (FP8) {
      // the codes widened exactly to bf16: the correction tiles' B operand
      uint64_t w = 0;
      if (rowvalid) w = *reinterpret_cast<const uint64_t*>(reinterpret_cast<const uint8_t*>(a.q) + qtok * D + d0);
      bf16x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = static_cast<__bf16>(fp8e4m3_to_f32((uint32_t)(w >> (8 * e)) & 0xFFu));
      qr[ks] = x;
    } else {
      bf16x8 x = {};
      if (rowvalid) x = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(a.q) + qtok * D + d0);
      qr[ks] = x;
    }
  }
  float qscale = 1.f;
  if constexpr (FP8) qscale = qvalid ? a.q_scale[(size_t)bh * Nb + I] : 0.f;
  // Retire every global load issued so far, so that the only vector-memory
  // operations in flight inside the main loop are the tile copies it counts.
  wait_vmcnt<0>();

  // ------------------------------------------------------------ LDS staging
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  auto tile_block = [&](int it) -> int {
    if constexpr (SPARSE) return ulist[it - nvirt] & 0xFFF;
    return it;
  };

  // Per-lane source offsets of the copies of a full tile (the same for the K
  // rows of an exact tile and the kbar rows of a correction tile, and for
  // both kinds of V^T tile).
  uint32_t koff[KI16], voff[VI];
#pragma unroll
  for (int i = 0; i < KI16; ++i) {
    const int P = (wave + NW * i) * 1024 + 16 * lane;
    const int row = P / C::KROW16, pc = (P % C::KROW16) / 16;
    koff[i] = row * C::KROW16 + swz<C::CPR16>(row, pc) * 16;
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int P = (wave + NW * i) * 1024 + 16 * lane;
    const int row = P / 128, pc = (P % 128) / 16;
    voff[i] = row * 128 + swz<8>(row, pc) * 16;
  }

  // Issue the LDS-DMA copies of tile `it` into stage `stg`.  Wave w's i-th
  // copy fills LDS bytes [(w + NW*i) KiB, +1 KiB) of the K or V^T buffer; lane
  // l writes 16 bytes at +16*l, i.e. physical chunk pc of row r, which holds
  // logical chunk pc ^ swz(r).  Rows past the end of the sequence re-read the
  // last valid row (finite data; those keys are masked).
  auto issue_tile = [&](int it, int stg) {
    const uint32_t kb = smem_base + stg * STAGE;
    const uint32_t vb = kb + C::KTILE;
    if (it < nvirt) {
      // 64 virtual keys: both bf16 halves of their key means (rows >= Nb
      // are zero) and, for the mean copies, the transposed value means
      const size_t row0 = ((size_t)bh * a.Nbp + 64 * it) * D;
      const uint64_t hbase = uniform_addr(a.kbar16 + row0), lbase = uniform_addr(a.kbarlo16 + row0);
#pragma unroll
      for (int i = 0; i < KI16; ++i) dma16s(koff[i], hbase, kb + (wave + NW * i) * 1024);
#pragma unroll
      for (int i = 0; i < KI16; ++i) dma16s(koff[i], lbase, kb + LO_OFF + (wave + NW * i) * 1024);
      if constexpr (!TAY) {
        const uint64_t vbase = uniform_addr(a.vbarT16 + ((size_t)bh * (a.Nbp / 64) + it) * D * 64);
#pragma unroll
        for (int i = 0; i < VI; ++i) dma16s(voff[i], vbase, vb + (wave + NW * i) * 1024);
      }
      return;
    }
    const int J = __builtin_amdgcn_readfirstlane(tile_block(it));
    constexpr bool k8 = FP8;
    // keys in position order: the caller's K, or its copy in tile order
    const void* kpos = (!FP8 && a.tm.on) ? static_cast<const void*>(a.kpos16) : a.k;
    const uint8_t* ksrc =
        reinterpret_cast<const uint8_t*>(kpos) + ((size_t)bh * N + (size_t)J * kBlock) * D * (FP8 ? 1 : 2);
    const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(a.vt16 + ((size_t)bh * Nb + J) * D * kBlock);
    const int kvalid = min(kBlock, N - J * kBlock);
    if (!k8 && kvalid == kBlock) {
      const uint64_t kbase = uniform_addr(ksrc), vbase = uniform_addr(vsrc);
#pragma unroll
      for (int i = 0; i < KI16; ++i) dma16s(koff[i], kbase, kb + (wave + NW * i) * 1024);
#pragma unroll
      for (int i = 0; i < VI; ++i) dma16s(voff[i], vbase, vb + (wave + NW * i) * 1024);
      return;
    }
    if (k8) {
#pragma unroll
      for (int i = 0; i < KI8; ++i) {
        const int P = (wave + NW * i) * 1024 + 16 * lane;
        const int row = P / C::KROW8, pc = (P % C::KROW8) / 16;
        const int src_row = min(row, kvalid - 1);
        dma16(ksrc + src_row * C::KROW8 + swz_any<C::CPR8>(row, pc) * 16, kb + (wave + NW * i) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KI16; ++i) {
        const int P = (wave + NW * i) * 1024 + 16 * lane;
        const int row = P / C::KROW16, pc = (P % C::KROW16) / 16;
        const int src_row = min(row, kvalid - 1);
        dma16(ksrc + src_row * C::KROW16 + swz<C::CPR16>(row, pc) * 16, kb + (wave + NW * i) * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int P = (wave + NW * i) * 1024 + 16 * lane;
      const int row = P / 128, pc = (P % 128) / 16;
      dma16(vsrc + row * 128 + swz<8>(row, pc) * 16, vb + (wave + NW * i) * 1024);
    }
  };

  // First-order values of correction tile `it` for this wave's query block:
  // rows [64 it, 64 it + 64) of V'[I] (16 KiB contiguous at D = 128), half a
  // tile per wave, issued before the next ring tile so that waiting for them
  // leaves that tile in flight.
  const uint32_t vps_base = (uint32_t)(uintptr_t)vps;
  auto issue_vprime = [&](int it) {
    constexpr int VPW = C::KTILE / 1024 / 2;
    const uint8_t* tile = reinterpret_cast<const uint8_t*>(a.vprime + (((size_t)bh * Nb + I) * a.Nbp + 64 * it) * D) +
                          qhalf * (C::KTILE / 2);
    const uint32_t off = 16 * lane;
#pragma unroll
    for (int i = 0; i < VPW; ++i)
      dma16s(off, uniform_addr(tile + 1024 * i), vps_base + qsel * C::KTILE + qhalf * (C::KTILE / 2) + 1024 * i);
  };

  // ----------------------------------------------------- online-softmax state
  f32x16 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = kMInit, l_run = 0.f;

  const float c2_base = a.scale * kLog2e;  // logits in log2 units
  const float log2_tail = log2f((float)ntail);

  // -------------------------------------------------------------- main loop
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < ntiles) issue_tile(s, s);
  // One tile: publish it, prefetch the tile ST-1 ahead, then S^T, softmax
  // and PV.  KIND selects the masks at compile time, so the plain exact
  // tiles -- nearly all of them -- carry no per-key selects.
  // STG >= 0: the ring stage of tile `it`, known at compile time (then the
  // LDS operand addresses are immediate offsets); -1: it % ST.
  auto step = [&](int it, auto kindc, auto stgc) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kindc)::value;
    constexpr int STG = decltype(stgc)::value;
    const int stg = STG >= 0 ? STG : it % ST;
    wait_tiles_ahead<LPT, ST - 2>(min(ST - 2, ntiles - 1 - it));
    __syncthreads();
    constexpr bool virt = KIND == kVirt;
    constexpr bool tv = TAY && virt;   // correction tile with first-order values
    if constexpr (tv) {
      if (qvalid) issue_vprime(it);
    }
    const bool ahead = it + ST - 1 < ntiles;
    if (ahead) issue_tile(it + ST - 1, STG >= 0 ? (STG + ST - 1) % ST : (it + ST - 1) % ST);
    // the value tile has landed (loads complete in order) and is visible to
    // both waves of the query block; every wave takes part
    auto values_ready = [&]() __attribute__((always_inline)) {
      if (ahead)
        wait_vmcnt<LPT>();
      else
        wait_vmcnt<0>();
      __syncthreads();
    };

    int J = 0;
    bool active = qvalid;
    if (!virt) {
      J = __builtin_amdgcn_readfirstlane(tile_block(it));
      if constexpr (SPARSE) active = active && ((ulist[it - nvirt] >> (12 + qsel)) & 1);
    }
    if (!active) {
      if constexpr (tv) values_ready();
      return;
    }

    // ---- the tile in two halves of 32 keys (kt = 0, 1): each half's scores
    // S^T = K Q^T, its weights and its part of O^T += V^T P^T.  The weights of
    // one half are computed between the matrix products of the other, so
    // that the vector ALU and the matrix core work side by side:
    //   region 1: S^T of half 0, then S^T of half 1 || weights of half 0
    //   region 2: PV of half 0                      || weights of half 1
    //   region 3: PV of half 1
    // Operands are read from LDS NPRE products ahead, and the source order is
    // pinned with scheduling barriers.
    const uint8_t* Kb = smem + stg * STAGE;
    const uint8_t* Vb = Kb + C::KTILE;
    float c2 = c2_base * qscale;
    constexpr bool k8 = FP8 && !virt;
    if constexpr (k8) c2 *= scalar_load_f32(a.k_scale + ((size_t)bh * Nb + J));
    constexpr int KS = C::KS, DT = C::DT;
    // products of S^T per half: D/16 bf16 MFMAs (K = 16); twice as many for
    // the correction tiles (the high and the low bf16 half of each key mean
    // against the same bf16 Q, summed in float32); or D/64 fp8 ones
    // (v_mfma_f32_32x32x64_f8f6f4, K = 64, twice the bf16 rate)
    constexpr int NS = k8 ? D / 64 : (virt ? 2 * KS : KS);
    constexpr int NPRE = 4;               // V^T operands in flight
    constexpr int NPK = k8 ? 2 : NPRE;    // K operands in flight
    constexpr int PB = 8 / (2 * DT);      // weight pairs per product in region 2
    using KOp = typename std::conditional<k8, i32x8, bf16x8>::type;
    auto kop = [&](int i) __attribute__((always_inline)) {  // operand of product i of region 1
      const int kt = i / NS, m = i % NS;
      const int krow = 32 * kt + kperm(l32);
      if constexpr (virt) {
        const uint8_t* half = Kb + (m < KS ? 0 : LO_OFF);
        return *reinterpret_cast<const bf16x8*>(half + krow * C::KROW16 + swz<C::CPR16>(krow, 2 * (m % KS) + h) * 16);
      }
      if constexpr (k8) {
        // 32 codes: dims [64m + 32h, +32) of key row krow, two 16-byte chunks
        const uint8_t* row = Kb + krow * C::KROW8;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(row + swz_any<C::CPR8>(krow, 4 * m + 2 * h) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(row + swz_any<C::CPR8>(krow, 4 * m + 2 * h + 1) * 16);
        i32x8 k;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k[e] = (int)lo[e];
          k[4 + e] = (int)hi[e];
        }
        return k;
      } else {
        return *reinterpret_cast<const bf16x8*>(Kb + krow * C::KROW16 + swz<C::CPR16>(krow, 2 * m + h) * 16);
      }
    };
    auto vop = [&](int i) __attribute__((always_inline)) {  // V^T operand of product i of regions 2-3
      const int k4 = i / DT, dt = i % DT;
      const int vrow = 32 * dt + l32;
      return *reinterpret_cast<const bf16x8*>(Vb + vrow * 128 + swz<8>(vrow, 2 * k4 + h) * 16);
    };

    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
    bf16x8 pb[4];
    float rs[2] = {0.f, 0.f};
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    const float inv_c2 = 1.f / c2;
    // Elements r, r+1 of half kt: the tile kind's masks and log-multiplicities
    // (applied to the raw scores, c2 > 0, and written back), then the bf16
    // weights 2^(s*c2 - m) and their sum.  Element r of half kt holds key
    // 32kt + 8h + j(r), j(r) = r for r < 8 and r + 8 above.  The masks are
    // applied once (MASK), not again when the weights are redone.
    auto w_pair = [&](int kt, int r, float negm, auto maskc) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(maskc)::value;
#pragma unroll
      for (int e = 0; e < 2 && MASK; ++e) {
        const int j = (r + e) < 8 ? (r + e) : (r + e) + 8;
        if constexpr (KIND == kVirt) {
          // virtual key J = 64*it + 32kt + 8h + j: live iff this query block
          // skips J; weight log2(n_J) = 6, or log2 of the tail's size
          const uint64_t bits = skipbits[qsel * (kMaxNb / 64) + it];
          const uint32_t lb = (uint32_t)(bits >> (32 * kt + 8 * h));
          const int jt = (Nb - 1) - 64 * it - 32 * kt - 8 * h;
          const bool live = (lb >> j) & 1u;
          const float w = (j == jt) ? log2_tail : 6.0f;
          s[kt][r + e] = live ? fmaf(w, inv_c2, s[kt][r + e]) : kNegInf;
        } else if constexpr (KIND == kTail) {
          if (j >= ntail - 32 * kt - 8 * h) s[kt][r + e] = kNegInf;
        }
      }
      const __bf16 b0 = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[kt][r], c2, negm)));
      const __bf16 b1 = static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(s[kt][r + 1], c2, negm)));
      pb[2 * kt + (r >> 3)][r & 7] = b0;
      pb[2 * kt + (r >> 3)][(r & 7) + 1] = b1;
      const bf16x2 pair = {b0, b1};
      rs[kt] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, rs[kt], false);
    };
    auto raise_max = [&](float mt) __attribute__((always_inline)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = (mn == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
    };
    // No per-tile maximum: the weights are taken against the maximum in use
    // as it stands, and only a half in which some row's weights exceed 2^64
    // or are not finite -- its maximum lies more than 64 above the one in use
    // (log2 units), as on a row's first tile, where the maximum in use is
    // kMInit -- raises it and is redone.  Exact: numerator and denominator
    // share the maximum, and weights up to 2^64 keep their relative precision
    // in bf16 and in the fp32 sums (masked keys give 2^-inf = 0).
    auto settle = [&](int kt) __attribute__((always_inline)) {
      if (__builtin_expect(__any(!(rs[kt] <= kWeightMax)), 0)) {
        float mt = s[kt][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[kt][r]);
        raise_max(xor32_max(mt) * c2);
        rs[kt] = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) w_pair(kt, r, -m_run, std::false_type{});
      }
      l_run += rs[kt];
    };
    auto mfma_s = [&](const KOp& ka, int m, f32x16& c) __attribute__((always_inline)) {
      if constexpr (k8)
        // format codes 0, 0: both operands fp8 e4m3; no block-exponent scales
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, q8[m], c, 0, 0, 0, 0, 0, 0);
      else
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qr[m], c, 0, 0, 0);
    };

    // region 1
    KOp kb[NPK];
    bf16x8 vb[NPRE];
#pragma unroll
    for (int i = 0; i < NPK; ++i) kb[i] = kop(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * NS; ++i) {
      const int kt = i / NS;
      mfma_s(kb[i % NPK], virt ? (i % NS) % KS : i % NS, s[kt]);
      if (i + NPK < 2 * NS) {
        kb[i % NPK] = kop(i + NPK);
      } else if constexpr (!tv) {
        // the first V^T operands of region 2, spread over the last products
#pragma unroll
        for (int v = (i + NPK - 2 * NS) * NPRE / NPK; v < (i + NPK - 2 * NS + 1) * NPRE / NPK; ++v) vb[v] = vop(v);
      }
      if (i >= NS) {
        // the 8 weight pairs of half 0 spread over the products of half 1
        const float negm = -m_run;
#pragma unroll
        for (int p = (i - NS) * 8 / NS; p < (i - NS + 1) * 8 / NS; ++p) w_pair(0, 2 * p, negm, std::true_type{});
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    settle(0);

    if constexpr (tv) {
      // first-order values: key rows in LDS, gathered 8 keys per operand
      // (lane: value column d = 32 dt + l32 of keys 16 k4 + 8 h + e)
      values_ready();
      const __bf16* vq = reinterpret_cast<const __bf16*>(vps + qsel * C::KTILE) + 8 * h * D + l32;
      auto pv_gather = [&](int k4) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          bf16x8 va;
#pragma unroll
          for (int e = 0; e < 8; ++e) va[e] = vq[(16 * k4 + e) * D + 32 * dt];
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[k4], acc[dt], 0, 0, 0);
        }
      };
      pv_gather(0);
      pv_gather(1);
      {
        const float negm = -m_run;
#pragma unroll
        for (int r = 0; r < 16; r += 2) w_pair(1, r, negm, std::true_type{});
      }
      settle(1);
      pv_gather(2);
      pv_gather(3);
    } else {
      // region 2
      {
        const float negm = -m_run;
#pragma unroll
        for (int i = 0; i < 2 * DT; ++i) {
          acc[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i % NPRE], pb[i / DT], acc[i % DT], 0, 0, 0);
          vb[i % NPRE] = vop(i + NPRE);
#pragma unroll
          for (int p = 0; p < PB; ++p) w_pair(1, 2 * (i * PB + p), negm, std::true_type{});
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      settle(1);
      // region 3
#pragma unroll
      for (int i = 2 * DT; i < 4 * DT; ++i) {
        acc[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i % NPRE], pb[i / DT], acc[i % DT], 0, 0, 0);
        if (i + NPRE < 4 * DT) vb[i % NPRE] = vop(i + NPRE);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    };
  // virtual (correction) tiles first, then the exact tiles of the union list
  // in key order, the ragged last key block -- always last -- on its own
  const bool has_tail = ntiles > nvirt && ntail < kBlock && tile_block(ntiles - 1) == Nb - 1;
  // tiles [it0, it1) of one kind; with a two-stage ring in pairs, so that
  // each copy of the body knows its stage
  auto run = [&](int it0, int it1, auto kindc) __attribute__((always_inline)) {
    if constexpr (ST == 2) {
      int it = it0;
      if (it < it1 && (it & 1)) step(it++, kindc, std::integral_constant<int, 1>{});
      for (; it + 1 < it1; it += 2) {
        step(it, kindc, std::integral_constant<int, 0>{});
        step(it + 1, kindc, std::integral_constant<int, 1>{});
      }
      if (it < it1) step(it, kindc, std::integral_constant<int, 0>{});
    } else {
      for (int it = it0; it < it1; ++it) step(it, kindc, std::integral_constant<int, -1>{});
    }
  };
  run(0, nvirt, std::integral_constant<int, kVirt>{});
  run(nvirt, ntiles - (has_tail ? 1 : 0), std::integral_constant<int, kPlain>{});
  if (has_tail) step(ntiles - 1, std::integral_constant<int, kTail>{}, std::integral_constant<int, -1>{});

  // --------------------------------------------------------------- 4. epilogue
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (rowvalid) {
    const float inv = 1.f / lt;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.o) + qtok * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        u32x2 w;
        w[0] = (uint32_t)f32_to_bf16_bits(acc[dt][4 * g + 0] * inv) |
               ((uint32_t)f32_to_bf16_bits(acc[dt][4 * g + 1] * inv) << 16);
        w[1] = (uint32_t)f32_to_bf16_bits(acc[dt][4 * g + 2] * inv) |
               ((uint32_t)f32_to_bf16_bits(acc[dt][4 * g + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    }
    if (h == 0) a.lse[qtok] = (m_run + __log2f(lt)) * kLn2;
  }
  if constexpr (!SPARSE) break;
  // every wave is done with the group's LDS before the next one is taken
  __syncthreads();
  }
}

#ifndef SA_QB
#define SA_QB 4
#endif
#ifndef SA_STAGES
#define SA_STAGES 2
#endif

// Persistent workgroups for the sparse kernel: as many as the device keeps
// resident at once (one per compute unit, two at D = 64).
int resident_groups(int per_cu) {
  static int ncu[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * per_cu;
  if (ncu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    ncu[dev] = n;
  }
  return ncu[dev] * per_cu;
}

template <int D, bool FP8>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  // D = 64 tiles are half the size: two query blocks per workgroup keep at
  // least one DMA copy per wave and two workgroups per CU
  constexpr int QB = D == 64 ? 2 : SA_QB;
  constexpr int STG = SA_STAGES;
  const int ngroups = (a.Nb + QB - 1) / QB;
  const int G = a.BH * ngroups;
  if (!a.sparse) {
    hipLaunchKernelGGL((attn_kernel<D, false, FP8, QB, STG>), dim3((unsigned)G), dim3(128 * QB), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(reset_sched, dim3(1), dim3(64), 0, st, a.sched);
  const dim3 grid((unsigned)std::min(G, resident_groups(QB == 2 ? 2 : 1)));
  if (a.vprime)
    // the first-order value tiles take 64 KB of LDS: two ring stages
    hipLaunchKernelGGL((attn_kernel<D, true, FP8, QB, 2, true>), grid, dim3(128 * QB), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<D, true, FP8, QB, STG>), grid, dim3(128 * QB), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st) {
  if (a.BH == 0 || a.N == 0) return hipSuccess;
  const bool fp8 = a.qk_elt == ELT_FP8;
  if (a.D == 64) return fp8 ? launch_d<64, true>(a, st) : launch_d<64, false>(a, st);
  return fp8 ? launch_d<128, true>(a, st) : launch_d<128, false>(a, st);
}

}  // namespace sa
