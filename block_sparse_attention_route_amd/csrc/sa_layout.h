// Workspace layout of libsa_route (host and device).  All sections start on
// 256-byte boundaries.  BH = B*H, Nb = ceil(N/64), Nbp = Nb rounded up to 64.
//
//   qbar    float [BH][Nb][D]         block means of Q (fp8: dequantised)
//   kbar    float [BH][Nb][D]         block means of K
//   vbar    float [BH][Nb][D]         block means of V
//   kbar16  bf16  [BH][Nbp][D]        bf16(kbar), rows >= Nb zero       (bf16 V only)
//   vbarT16 bf16  [BH][Nbp/64][D][64] bf16(vbar) grouped 64 blocks at a
//                                     time and transposed, cols >= Nb zero (bf16 V only)
//   vt16    bf16  [BH][Nb][D][64]     V regrouped per 64-key block and
//                                     transposed (d-major), keys >= N zero (bf16 V only)
//
// The dense path uses only vt16.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sa {

constexpr int kBlock = 64;
constexpr int kMaxNb = 4096;

struct WsLayout {
  size_t qbar, kbar, vbar, kbar16, vbarT16, vt16, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline WsLayout ws_layout(int64_t BH, int64_t N, int64_t D, bool v_bf16,
                                              bool dense_only) {
  const int64_t Nb = (N + kBlock - 1) / kBlock;
  const int64_t Nbp = (Nb + 63) / 64 * 64;
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  if (!dense_only) {
    L.qbar = take((size_t)(BH * Nb * D) * 4);
    L.kbar = take((size_t)(BH * Nb * D) * 4);
    L.vbar = take((size_t)(BH * Nb * D) * 4);
    if (v_bf16) {
      L.kbar16 = take((size_t)(BH * Nbp * D) * 2);
      L.vbarT16 = take((size_t)(BH * Nbp * D) * 2);
    }
  }
  if (v_bf16) L.vt16 = take((size_t)(BH * Nb * D * kBlock) * 2);
  L.total = off;
  return L;
}

}  // namespace sa
