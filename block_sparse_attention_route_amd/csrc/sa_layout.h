// Workspace layout of libsa_route (host and device).  All sections start on
// 256-byte boundaries.  BH = B*H, Nb = ceil(N/64), Nbp = Nb rounded up to 64.
//
//   qbar    float [BH][Nb][D]         block means of Q (fp8: dequantised)
//   kbar    float [BH][Nb][D]         block means of K
//   vbar    float [BH][Nb][D]         block means of V
//   kbar16  bf16  [2][BH][Nbp][D]     kbar in two bf16 halves: [0] = bf16(kbar),
//                                     [1] = bf16(kbar - [0]); rows >= Nb zero (bf16 V only)
//   vbarT16 bf16  [BH][Nbp/64][D][64] bf16(vbar) grouped 64 blocks at a
//                                     time and transposed, cols >= Nb zero (bf16 V only)
//   vt16    bf16  [BH][Nb][D][64]     V regrouped per 64-key block and
//                                     transposed (d-major), keys >= N zero (bf16 V only)
//   kpos16  bf16  [BH][N][D]          K in block (position) order; only with a
//                                     3-D tile order (bf16 K only)
//   sched   int   [64]                group counters of the sparse attention
//                                     kernel's persistent workgroups
//   vprime  bf16  [S][Nb][Nbp][D]     first-order values of the skipped blocks
//                                     of a slab of S heads, per query block I
//                                     and key block J, rows J >= Nb zero; only
//                                     with correction mode 2 (fp32 inputs:
//                                     float [S][Nb][Nb][D]).  S = first_order_slab()
//
// The dense path uses only vt16.  Blocks are formed over positions: position
// i is token i in the raster order, or token_of(i) in the 3-D tile order.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sa {

constexpr int kBlock = 64;
constexpr int kMaxNb = 4096;

struct WsLayout {
  size_t qbar, kbar, vbar, kbar16, vbarT16, vt16, kpos16, sched, vprime, total;
};

// Position -> token map of the 3-D tile order.  Full tiles of tt x th x tw =
// 64 tokens come first, in raster order of their (frame, row, column) tile
// coordinates, tokens inside a tile in (t, y, x) raster order; then every
// token outside the full tiles, in the frame-major raster order.  on == 0 is
// the raster order itself.  Filled on the host (make_tile_map).
struct TileMap {
  int on;
  int Hg, Wg;        // grid rows and columns of a frame
  int tt, th, tw;    // tile extent, tt * th * tw == 64
  int nfy, nfx;      // full tiles along y and x
  int nfull;         // full tiles in total
  int Tf, Hf, Wf;    // extent covered by full tiles
};

__host__ __device__ inline TileMap make_tile_map(int T, int Hg, int Wg, int tt, int th, int tw) {
  TileMap m{};
  m.on = (tt > 0) ? 1 : 0;
  m.Hg = Hg;
  m.Wg = Wg;
  m.tt = tt > 0 ? tt : 1;
  m.th = th > 0 ? th : 1;
  m.tw = tw > 0 ? tw : 1;
  m.nfy = Hg / m.th;
  m.nfx = Wg / m.tw;
  const int nfz = T / m.tt;
  m.nfull = nfz * m.nfy * m.nfx;
  m.Tf = nfz * m.tt;
  m.Hf = m.nfy * m.th;
  m.Wf = m.nfx * m.tw;
  return m;
}

// Token index (within one head) at position pos.
__host__ __device__ inline int token_of(const TileMap& m, int pos) {
  if (!m.on) return pos;
  if (pos < 64 * m.nfull) {
    const int f = pos >> 6, w = pos & 63;
    const int fx = f % m.nfx, fy = (f / m.nfx) % m.nfy, fz = f / (m.nfx * m.nfy);
    const int dx = w % m.tw, dy = (w / m.tw) % m.th, dz = w / (m.tw * m.th);
    return ((fz * m.tt + dz) * m.Hg + fy * m.th + dy) * m.Wg + fx * m.tw + dx;
  }
  const int r = pos - 64 * m.nfull;           // rank among the uncovered tokens
  const int wl = m.Wg - m.Wf;                 // uncovered columns of a covered row
  const int lf = m.Hf * wl + (m.Hg - m.Hf) * m.Wg;  // uncovered tokens of a frame t < Tf
  if (r < m.Tf * lf) {
    const int t = r / lf, r2 = r - t * lf;
    int y, x;
    if (r2 < m.Hf * wl) {
      y = r2 / wl;
      x = m.Wf + r2 % wl;
    } else {
      const int r3 = r2 - m.Hf * wl;
      y = m.Hf + r3 / m.Wg;
      x = r3 % m.Wg;
    }
    return (t * m.Hg + y) * m.Wg + x;
  }
  return m.Tf * m.Hg * m.Wg + (r - m.Tf * lf);   // frames t >= Tf: all of them
}

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The first-order values are computed and consumed a slab of heads at a
// time: the fewest slabs of equal size (up to one head) whose values fit in
// kFirstOrderSlabBytes each -- or one head per slab where one head needs
// more.
constexpr size_t kFirstOrderSlabBytes = (size_t)8 << 30;

__host__ __device__ inline size_t first_order_head_bytes(int64_t N, int64_t D, bool v_bf16) {
  const int64_t Nb = (N + kBlock - 1) / kBlock;
  const int64_t Nbp = (Nb + 63) / 64 * 64;
  return v_bf16 ? (size_t)(Nb * Nbp * D) * 2 : (size_t)(Nb * Nb * D) * 4;
}

__host__ __device__ inline int64_t first_order_slab(int64_t BH, int64_t N, int64_t D, bool v_bf16) {
  if (BH < 1) return 0;
  const size_t per = first_order_head_bytes(N, D, v_bf16);
  int64_t fit = per > 0 ? (int64_t)(kFirstOrderSlabBytes / per) : BH;
  if (fit < 1) fit = 1;
  const int64_t slabs = (BH + fit - 1) / fit;
  return (BH + slabs - 1) / slabs;
}

__host__ __device__ inline WsLayout ws_layout(int64_t BH, int64_t N, int64_t D, bool v_bf16,
                                              bool dense_only, bool tiled = false, bool first_order = false) {
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
      L.kbar16 = take((size_t)(2 * BH * Nbp * D) * 2);
      L.vbarT16 = take((size_t)(BH * Nbp * D) * 2);
    }
  }
  if (v_bf16) L.vt16 = take((size_t)(BH * Nb * D * kBlock) * 2);
  if (tiled && v_bf16 && !dense_only) L.kpos16 = take((size_t)(BH * N * D) * 2);
  if (!dense_only) L.sched = take(256);
  if (first_order && !dense_only)
    L.vprime = take((size_t)first_order_slab(BH, N, D, v_bf16) * first_order_head_bytes(N, D, v_bf16));
  L.total = off;
  return L;
}

}  // namespace sa
