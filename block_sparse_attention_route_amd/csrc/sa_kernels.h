// Host-side launchers of the libsa_route kernels (internal; the public ABI
// is include/sa_route.h).  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_layout.h"

namespace sa {

enum Elt : int { ELT_F32 = 0, ELT_BF16 = 1, ELT_FP8 = 2 };

// Fused Q/K producer in front of the pool (per-head RMS norm with gain,
// 3-D rotary embedding, bf16 rounding): the transformed rows are written to
// q_out / k_out and pooled in place of the inputs.
struct ProArgs {
  bool on;
  const float* q_gain;   // [D]
  const float* k_gain;   // [D]
  uint16_t* q_out;       // [BH][N][D] bf16, token order
  uint16_t* k_out;
  float eps, base;
  int T, Hg, Wg;
};

struct PoolArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;  // [BH][Nb] (fp8 only)
  const float* k_scale;
  int BH, N, Nb, Nbp, D;
  int qk_elt, v_elt;
  bool vt_only;          // dense path: only regroup V
  float* qbar;
  float* kbar;
  float* vbar;
  uint16_t* kbar16;
  uint16_t* vbarT16;
  uint16_t* vt16;
  TileMap tm;            // position -> token order (on == 0: raster)
  uint16_t* kpos16;      // K in position order, written when tm.on (bf16 K)
  ProArgs pro;           // producer step fused in front (pro.on)
  int* sched;            // the attention kernel's group counters [64], zeroed here (or null)
};

// First-order values of the skipped blocks (correction mode 2): the bf16
// path (vprime) or the float32 path (vprime32), whichever is set.
struct TaylorArgs {
  const uint16_t* k;     // bf16: [BH][N][D] K in position order (the caller's K, or kpos16)
  const float* qbar;     // [BH][Nb][D]
  const float* kbar;
  const float* vbar;
  const uint16_t* vt16;  // bf16: [BH][Nb][D][64]
  uint16_t* vprime;      // bf16: [BH][Nb][Nbp][D]
  int BH, N, Nb, Nbp, D;
  float scale;           // softmax scale s
  const float* kf;       // float32: [BH][N][D] K and V in token order, read through tm
  const float* vf;
  TileMap tm;
  float* vprime32;       // float32: [BH][Nb][Nb][D]
  const uint8_t* k8;     // fp8 e4m3 K codes [BH][N][D] (with k_scale), else null
  const float* k_scale;  // [BH][Nb]
};

struct RouteArgs {
  const float* qbar;
  const float* kbar;
  int BH, Nb, D;
  float scale, tau;
  int topk;              // > 0: fixed budget of key blocks per query block
  uint8_t* mask;         // [BH][Nb][Nb]
  int32_t* kept;         // [BH][Nb] or null
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;         // original V (fp32 path)
  const float* q_scale;
  const float* k_scale;
  const float* qbar;
  const float* kbar;
  const float* vbar;
  const uint16_t* kbar16;    // bf16(kbar) [BH][Nbp][D]
  const uint16_t* kbarlo16;  // bf16(kbar - bf16(kbar)) [BH][Nbp][D]
  const uint16_t* vbarT16;
  const uint16_t* vt16;
  TileMap tm;            // position -> token order (on == 0: raster)
  const uint16_t* kpos16;  // K in position order when tm.on (bf16 K)
  void* o;
  float* lse;
  int32_t* kept;
  int BH, N, Nb, Nbp, D;
  int qk_elt, v_elt;
  float scale;           // softmax scale s
  float tau;
  int topk;              // > 0: fixed budget of key blocks per query block
  int correction;
  bool sparse;           // false: dense attention over all blocks
  const uint16_t* vprime;  // correction mode 2: first-order values, else null
  const float* vprime32;   // the same for the float32 path
  int* sched;              // sparse: 8 per-XCD group counters (zeroed by the launcher)
};

hipError_t launch_pool(const PoolArgs& a, hipStream_t st);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
hipError_t launch_taylor(const TaylorArgs& a, hipStream_t st);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st);

}  // namespace sa
