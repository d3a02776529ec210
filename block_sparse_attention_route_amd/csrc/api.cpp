// C ABI of libsa_route (declared in include/sa_route.h): argument validation,
// workspace carve-up and kernel launches.  Every check runs on the host
// before anything is enqueued; a failed check returns a status and leaves a
// message in a thread-local buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "sa_kernels.h"
#include "sa_layout.h"
#include "sa_route.h"

#define SA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";
thread_local sa_status g_status = SA_OK;

sa_status fail(sa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  g_status = s;
  return s;
}

sa_status ok() {
  g_err[0] = '\0';
  g_status = SA_OK;
  return SA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Req {
  int64_t B, H, BH, N, Nb, Nbp;
  int D;
  int qk, v;
  bool empty;
  float scale, tau;
  int topk;
  int correction;
  int T, Hg, Wg;
  bool dense;
  sa::TileMap tm;
  sa::WsLayout ws;
};

sa_status check_shape_inputs(const sa_shape* sh, const sa_inputs* in, Req* r, bool dense,
                             bool ptrs = true) {
  if (!sh) return fail(SA_ERR_NULL, "shape is NULL");
  if (!in) return fail(SA_ERR_NULL, "inputs is NULL");
  if (sh->B < 0 || sh->H < 0 || sh->N < 0 || sh->T < 0 || sh->Hg < 0 || sh->Wg < 0)
    return fail(SA_ERR_SHAPE, "negative dimension");
  if (sh->D != 64 && sh->D != 128) return fail(SA_ERR_SHAPE, "D must be 64 or 128 (got %d)", sh->D);
  const int64_t grid = (int64_t)sh->T * sh->Hg * sh->Wg;
  if (grid != sh->N)
    return fail(SA_ERR_SHAPE, "N (%d) != T*Hg*Wg (%lld)", sh->N, (long long)grid);
  if (sh->N > SA_MAX_N) return fail(SA_ERR_SHAPE, "N (%d) exceeds SA_MAX_N (%d)", sh->N, SA_MAX_N);
  const int qk = in->qk_dtype, v = in->v_dtype;
  const bool pair_ok = (qk == SA_F32 && v == SA_F32) || (qk == SA_BF16 && v == SA_BF16) ||
                       (qk == SA_FP8_E4M3 && v == SA_BF16);
  if (!pair_ok) return fail(SA_ERR_DTYPE, "unsupported dtype pair (qk=%d, v=%d)", qk, v);
  const bool fp8 = qk == SA_FP8_E4M3;
  r->B = sh->B;
  r->H = sh->H;
  r->BH = (int64_t)sh->B * sh->H;
  r->N = sh->N;
  r->D = sh->D;
  r->Nb = (r->N + SA_BLOCK - 1) / SA_BLOCK;
  r->Nbp = (r->Nb + 63) / 64 * 64;
  r->qk = qk;
  r->v = v;
  r->empty = r->BH * r->N == 0;
  r->T = sh->T;
  r->Hg = sh->Hg;
  r->Wg = sh->Wg;
  r->dense = dense;
  r->tm = sa::make_tile_map(sh->T, sh->Hg, sh->Wg, 0, 0, 0);
  if (r->BH > (int64_t)1 << 24) return fail(SA_ERR_SHAPE, "B*H too large");
  // every launch's grid has at most B*H*Nb workgroups: keep it a positive int
  if (r->BH * r->Nb > (int64_t)INT32_MAX)
    return fail(SA_ERR_SHAPE, "B*H*Nb (%lld) exceeds 2^31 - 1", (long long)(r->BH * r->Nb));
  r->ws = sa::ws_layout(r->BH, r->N, r->D, v == SA_BF16, dense);
  if (!ptrs) return SA_OK;  // sizing only: data pointers are not needed
  if (!fp8 && (in->q_scale || in->k_scale))
    return fail(SA_ERR_DTYPE, "q_scale/k_scale given for a non-fp8 qk_dtype");
  if (r->empty) return SA_OK;
  if (!in->q || !in->k || !in->v) return fail(SA_ERR_NULL, "q, k or v is NULL");
  if (fp8 && (!in->q_scale || !in->k_scale))
    return fail(SA_ERR_DTYPE, "fp8 qk_dtype needs q_scale and k_scale");
  if (!aligned(in->q, 16) || !aligned(in->k, 16) || !aligned(in->v, 16))
    return fail(SA_ERR_ALIGN, "q, k and v must be 16-byte aligned");
  if (fp8 && (!aligned(in->q_scale, 4) || !aligned(in->k_scale, 4)))
    return fail(SA_ERR_ALIGN, "scales must be 4-byte aligned");
  return SA_OK;
}

sa_status check_params(const sa_params* p, Req* r) {
  if (!p) return fail(SA_ERR_NULL, "params is NULL");
  if (p->block != SA_BLOCK) return fail(SA_ERR_PARAM, "block must be %d (got %d)", SA_BLOCK, p->block);
  if (p->topk < 0) return fail(SA_ERR_PARAM, "topk must be >= 0 (got %d)", p->topk);
  if (p->topk == 0 && (std::isnan(p->tau) || p->tau < 0.f))
    return fail(SA_ERR_PARAM, "tau must be >= 0 or +inf");
  if (p->correction < 0 || p->correction > 2) return fail(SA_ERR_PARAM, "correction must be 0, 1 or 2");
  if (!std::isfinite(p->scale)) return fail(SA_ERR_PARAM, "scale must be finite");
  const int tt = p->tile_t, th = p->tile_h, tw = p->tile_w;
  if (tt != 0 || th != 0 || tw != 0) {
    if (tt < 1 || th < 1 || tw < 1 || (int64_t)tt * th * tw != SA_BLOCK)
      return fail(SA_ERR_PARAM, "tile (%d, %d, %d) must be all 0 or positive with product %d", tt, th, tw,
                  SA_BLOCK);
    if (r->qk == SA_FP8_E4M3)
      return fail(SA_ERR_UNSUPPORTED, "a 3-D tile order needs bf16 or fp32 Q/K (fp8 block scales "
                  "belong to raster blocks)");
    r->tm = sa::make_tile_map(r->T, r->Hg, r->Wg, tt, th, tw);
  }
  r->ws = sa::ws_layout(r->BH, r->N, r->D, r->v == SA_BF16, r->dense, r->tm.on != 0, p->correction == 2);
  r->tau = p->tau;
  r->topk = p->topk;
  r->correction = p->correction;
  r->scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)r->D);
  return SA_OK;
}

sa_status check_ws(const void* ws, size_t ws_bytes, const Req& r) {
  if (r.ws.total == 0) return SA_OK;
  if (!ws) return fail(SA_ERR_NULL, "workspace is NULL");
  if (!aligned(ws, 16)) return fail(SA_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (ws_bytes < r.ws.total)
    return fail(SA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, r.ws.total);
  return SA_OK;
}

sa_status check_out(const void* o, const float* lse, const int32_t* kept) {
  if (!o || !lse) return fail(SA_ERR_NULL, "o or lse is NULL");
  if (!aligned(o, 16)) return fail(SA_ERR_ALIGN, "o must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(SA_ERR_ALIGN, "lse must be 4-byte aligned");
  if (kept && !aligned(kept, 4)) return fail(SA_ERR_ALIGN, "kept must be 4-byte aligned");
  return SA_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

sa::PoolArgs pool_args(const Req& r, const sa_inputs* in, void* ws, bool vt_only) {
  sa::PoolArgs a{};
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.q_scale = in->q_scale;
  a.k_scale = in->k_scale;
  a.BH = (int)r.BH;
  a.N = (int)r.N;
  a.Nb = (int)r.Nb;
  a.Nbp = (int)r.Nbp;
  a.D = r.D;
  a.qk_elt = r.qk;
  a.v_elt = r.v;
  a.vt_only = vt_only;
  if (!vt_only) {
    a.qbar = at<float>(ws, r.ws.qbar);
    a.kbar = at<float>(ws, r.ws.kbar);
    a.vbar = at<float>(ws, r.ws.vbar);
    if (r.v == SA_BF16) {
      a.kbar16 = at<uint16_t>(ws, r.ws.kbar16);
      a.vbarT16 = at<uint16_t>(ws, r.ws.vbarT16);
    }
  }
  if (r.v == SA_BF16) a.vt16 = at<uint16_t>(ws, r.ws.vt16);
  if (!vt_only) {
    a.tm = r.tm;
    a.sched = at<int>(ws, r.ws.sched);
    if (r.tm.on && r.qk == SA_BF16) a.kpos16 = at<uint16_t>(ws, r.ws.kpos16);
  }
  return a;
}

sa::AttnArgs attn_args(const Req& r, const sa_inputs* in, void* o, float* lse, int32_t* kept,
                       void* ws, bool sparse) {
  sa::AttnArgs a{};
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.q_scale = in->q_scale;
  a.k_scale = in->k_scale;
  if (sparse) {
    a.qbar = at<float>(ws, r.ws.qbar);
    a.kbar = at<float>(ws, r.ws.kbar);
    a.vbar = at<float>(ws, r.ws.vbar);
    if (r.v == SA_BF16) {
      a.kbar16 = at<uint16_t>(ws, r.ws.kbar16);
      a.kbarlo16 = a.kbar16 + (size_t)r.BH * r.Nbp * r.D;
      a.vbarT16 = at<uint16_t>(ws, r.ws.vbarT16);
    }
  }
  if (r.v == SA_BF16) a.vt16 = at<uint16_t>(ws, r.ws.vt16);
  if (sparse) {
    a.tm = r.tm;
    a.sched = at<int>(ws, r.ws.sched);
    if (r.tm.on && r.qk == SA_BF16) a.kpos16 = at<uint16_t>(ws, r.ws.kpos16);
    if (r.correction == 2) {
      if (r.qk == SA_F32)
        a.vprime32 = at<float>(ws, r.ws.vprime);
      else
        a.vprime = at<uint16_t>(ws, r.ws.vprime);
    }
  }
  a.o = o;
  a.lse = lse;
  a.kept = kept;
  a.BH = (int)r.BH;
  a.N = (int)r.N;
  a.Nb = (int)r.Nb;
  a.Nbp = (int)r.Nbp;
  a.D = r.D;
  a.qk_elt = r.qk;
  a.v_elt = r.v;
  a.scale = r.scale;
  a.tau = r.tau;
  a.topk = r.topk;
  a.correction = r.correction;
  a.sparse = sparse;
  return a;
}

sa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// The first-order correction's values per (query block, key block) of heads
// [bh0, bh0 + nbh), from the pooled means in the workspace and K (bf16: its
// position-order copy with a 3-D tile order, V from the regrouped copy; fp32:
// K and V read through the order), into the workspace's slab of values.
sa_status run_taylor(const Req& r, const void* k, const void* v, const float* k_scale, void* ws,
                     int64_t bh0, int64_t nbh, hipStream_t st) {
  sa::TaylorArgs a{};
  const size_t mh = (size_t)bh0 * r.Nb * r.D;  // per-head offsets of the inputs
  const size_t th = (size_t)bh0 * r.N * r.D;
  a.qbar = at<float>(ws, r.ws.qbar) + mh;
  a.kbar = at<float>(ws, r.ws.kbar) + mh;
  a.vbar = at<float>(ws, r.ws.vbar) + mh;
  if (r.qk == SA_F32) {
    a.kf = static_cast<const float*>(k) + th;
    a.vf = static_cast<const float*>(v) + th;
    a.tm = r.tm;
    a.vprime32 = at<float>(ws, r.ws.vprime);
  } else {
    if (r.qk == SA_FP8_E4M3) {
      a.k8 = static_cast<const uint8_t*>(k) + th;   // fp8 Q/K have no 3-D tile order
      a.k_scale = k_scale + (size_t)bh0 * r.Nb;
    } else {
      a.k = static_cast<const uint16_t*>(r.tm.on ? at<uint16_t>(ws, r.ws.kpos16) : k) + th;
    }
    a.vt16 = at<uint16_t>(ws, r.ws.vt16) + (size_t)bh0 * r.Nb * r.D * SA_BLOCK;
    a.vprime = at<uint16_t>(ws, r.ws.vprime);
  }
  a.BH = (int)nbh;
  a.N = (int)r.N;
  a.Nb = (int)r.Nb;
  a.Nbp = (int)r.Nbp;
  a.D = r.D;
  a.scale = r.scale;
  return hip_status(sa::launch_taylor(a, st), "first-order values kernel launch");
}

sa_status run_pool(const Req& r, const sa_inputs* in, void* ws, hipStream_t st) {
  return hip_status(sa::launch_pool(pool_args(r, in, ws, false), st), "pool kernel launch");
}

// The arguments of one launch over heads [bh0, bh0 + nbh): every per-head
// tensor pointer moves to head bh0; the first-order values are slab-local.
sa::AttnArgs head_slab(sa::AttnArgs a, const Req& r, int64_t bh0, int64_t nbh) {
  const size_t nd = (size_t)bh0 * r.N * r.D, bd = (size_t)bh0 * r.Nb * r.D, pd = (size_t)bh0 * r.Nbp * r.D;
  const size_t qe = r.qk == SA_F32 ? 4 : r.qk == SA_BF16 ? 2 : 1, ve = r.v == SA_F32 ? 4 : 2;
  auto adv = [](const void* p, size_t bytes) -> const void* {
    return p ? static_cast<const uint8_t*>(p) + bytes : nullptr;
  };
  a.q = adv(a.q, nd * qe);
  a.k = adv(a.k, nd * qe);
  a.v = adv(a.v, nd * ve);
  if (a.q_scale) a.q_scale += (size_t)bh0 * r.Nb;
  if (a.k_scale) a.k_scale += (size_t)bh0 * r.Nb;
  if (a.qbar) a.qbar += bd;
  if (a.kbar) a.kbar += bd;
  if (a.vbar) a.vbar += bd;
  if (a.kbar16) a.kbar16 += pd;
  if (a.kbarlo16) a.kbarlo16 += pd;
  if (a.vbarT16) a.vbarT16 += pd;
  if (a.vt16) a.vt16 += bd * SA_BLOCK;
  if (a.kpos16) a.kpos16 += nd;
  a.o = static_cast<uint8_t*>(a.o) + nd * ve;
  a.lse += (size_t)bh0 * r.N;
  if (a.kept) a.kept += (size_t)bh0 * r.Nb;
  a.BH = (int)nbh;
  return a;
}

sa_status run_attn(const Req& r, const sa_inputs* in, void* o, float* lse, int32_t* kept, void* ws,
                   bool sparse, hipStream_t st) {
  const sa::AttnArgs a = attn_args(r, in, o, lse, kept, ws, sparse);
  auto launch = [&](const sa::AttnArgs& x) {
    return hip_status(r.qk == SA_F32 ? sa::launch_attn_f32(x, st) : sa::launch_attn_mfma(x, st),
                      "attention kernel launch");
  };
  if (!(sparse && r.correction == 2)) return launch(a);
  // first-order correction: per slab of heads, the values, then the attention
  const int64_t slab = sa::first_order_slab(r.BH, r.N, r.D, r.v == SA_BF16);
  for (int64_t bh0 = 0; bh0 < r.BH; bh0 += slab) {
    const int64_t nbh = std::min<int64_t>(slab, r.BH - bh0);
    sa_status s = run_taylor(r, in->k, in->v, in->k_scale, ws, bh0, nbh, st);
    if (s != SA_OK) return s;
    if ((s = launch(head_slab(a, r, bh0, nbh))) != SA_OK) return s;
  }
  return ok();
}

}  // namespace

// ---------------------------------------------------------------------------
// sa_forward_noalloc: sa_forward with the workspace in a static device array,
// for callers that cannot allocate.  Each device holds its own copy of the
// array; its device address is looked up once per device and kept.
static __device__ __align__(256) uint8_t scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sa_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

}  // namespace

SA_API sa_status sa_forward_noalloc(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                                    void* o, float* lse, int32_t* kept, void* stream) {
  Req r{};
  sa_status s;
  if ((s = check_shape_inputs(shape, in, &r, false)) != SA_OK) return s;
  if ((s = check_params(params, &r)) != SA_OK) return s;
  if (r.empty) return ok();
  if ((s = check_out(o, lse, kept)) != SA_OK) return s;
  if (r.ws.total > (size_t)SA_NOALLOC_SCRATCH_BYTES)
    return fail(SA_ERR_WORKSPACE, "sa_forward_noalloc: this call needs a %zu-byte workspace, above the %zu-byte "
                "static scratch (SA_NOALLOC_SCRATCH_BYTES); use sa_forward with a caller workspace",
                r.ws.total, (size_t)SA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != SA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if ((s = run_pool(r, in, ws, st)) != SA_OK) return s;
  return run_attn(r, in, o, lse, kept, ws, true, st);
}

SA_API int32_t sa_abi_version(void) { return SA_ABI_VERSION; }

SA_API const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL: a required pointer is NULL";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE: invalid shape";
    case SA_ERR_PARAM: return "SA_ERR_PARAM: invalid routing parameter";
    case SA_ERR_DTYPE: return "SA_ERR_DTYPE: unsupported dtype combination";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN: misaligned pointer";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE: workspace too small";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: not implemented";
    case SA_ERR_HIP: return "SA_ERR_HIP: HIP runtime error";
  }
  return "unknown sa_status";
}

SA_API const char* sa_last_error(void) { return g_err; }

SA_API sa_status sa_last_status(void) { return g_status; }

SA_API size_t sa_workspace_bytes(const sa_shape* shape, const sa_params* params, const sa_inputs* in) {
  Req r{};
  if (check_shape_inputs(shape, in, &r, false, false) != SA_OK) return 0;
  if (params) {
    if (check_params(params, &r) != SA_OK) return 0;
  }
  ok();
  return r.ws.total;
}

SA_API int64_t sa_first_order_slab_heads(const sa_shape* shape, const sa_inputs* in) {
  Req r{};
  if (check_shape_inputs(shape, in, &r, false, false) != SA_OK) return 0;
  ok();
  return r.BH == 0 ? 0 : sa::first_order_slab(r.BH, r.N, r.D, r.v == SA_BF16);
}

SA_API int32_t sa_budget_blocks(int32_t N, double sparsity) {
  if (N < 1 || !(sparsity >= 0.0) || !(sparsity < 1.0)) {
    fail(SA_ERR_PARAM, "budget needs N >= 1 and sparsity in [0, 1)");
    return 0;
  }
  ok();
  const int64_t Nb = ((int64_t)N + SA_BLOCK - 1) / SA_BLOCK;
  // the 1e-9 keeps a product that is an integer up to rounding at that integer
  const int64_t k = (int64_t)std::ceil((1.0 - sparsity) * (double)Nb - 1e-9);
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(k, Nb));
}

SA_API size_t sa_dense_workspace_bytes(const sa_shape* shape, const sa_inputs* in) {
  Req r{};
  if (check_shape_inputs(shape, in, &r, true, false) != SA_OK) return 0;
  ok();
  return r.ws.total;
}

SA_API sa_status sa_pool(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                         void* ws, size_t ws_bytes, void* stream) {
  Req r{};
  sa_status s;
  if ((s = check_shape_inputs(shape, in, &r, false)) != SA_OK) return s;
  if ((s = check_params(params, &r)) != SA_OK) return s;
  if (r.empty) return ok();
  if ((s = check_ws(ws, ws_bytes, r)) != SA_OK) return s;
  return run_pool(r, in, ws, (hipStream_t)stream);
}

SA_API sa_status sa_route(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                          uint8_t* mask, int32_t* kept, void* ws, size_t ws_bytes, void* stream) {
  Req r{};
  sa_status s;
  if ((s = check_shape_inputs(shape, in, &r, false)) != SA_OK) return s;
  if ((s = check_params(params, &r)) != SA_OK) return s;
  if (r.empty) return ok();
  if (!mask) return fail(SA_ERR_NULL, "mask is NULL");
  if (kept && !aligned(kept, 4)) return fail(SA_ERR_ALIGN, "kept must be 4-byte aligned");
  if ((s = check_ws(ws, ws_bytes, r)) != SA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if ((s = hip_status(sa::launch_pool(pool_args(r, in, ws, false), st), "pool kernel launch")) != SA_OK)
    return s;
  sa::RouteArgs a{};
  a.qbar = at<float>(ws, r.ws.qbar);
  a.kbar = at<float>(ws, r.ws.kbar);
  a.BH = (int)r.BH;
  a.Nb = (int)r.Nb;
  a.D = r.D;
  a.scale = r.scale;
  a.tau = r.tau;
  a.topk = r.topk;
  a.mask = mask;
  a.kept = kept;
  return hip_status(sa::launch_route(a, st), "route kernel launch");
}

SA_API sa_status sa_forward_pooled(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                                   void* o, float* lse, int32_t* kept, void* ws, size_t ws_bytes,
                                   void* stream) {
  Req r{};
  sa_status s;
  if ((s = check_shape_inputs(shape, in, &r, false)) != SA_OK) return s;
  if ((s = check_params(params, &r)) != SA_OK) return s;
  if (r.empty) return ok();
  if ((s = check_out(o, lse, kept)) != SA_OK) return s;
  if ((s = check_ws(ws, ws_bytes, r)) != SA_OK) return s;
  return run_attn(r, in, o, lse, kept, ws, true, (hipStream_t)stream);
}

SA_API sa_status sa_forward(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                            void* o, float* lse, int32_t* kept, void* ws, size_t ws_bytes,
                            void* stream) {
  Req r{};
  sa_status s;
  if ((s = check_shape_inputs(shape, in, &r, false)) != SA_OK) return s;
  if ((s = check_params(params, &r)) != SA_OK) return s;
  if (r.empty) return ok();
  if ((s = check_out(o, lse, kept)) != SA_OK) return s;
  if ((s = check_ws(ws, ws_bytes, r)) != SA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if ((s = run_pool(r, in, ws, st)) != SA_OK) return s;
  return run_attn(r, in, o, lse, kept, ws, true, st);
}

SA_API sa_status sa_qk_prologue(const sa_shape* shape, const sa_params* params, const sa_prologue* pro,
                                const sa_inputs* in, const float* q_gain, const float* k_gain, void* q_out,
                                void* k_out, void* ws, size_t ws_bytes, void* stream) {
  Req r{};
  sa_status s;
  if ((s = check_shape_inputs(shape, in, &r, false)) != SA_OK) return s;
  if ((s = check_params(params, &r)) != SA_OK) return s;
  if (!pro) return fail(SA_ERR_NULL, "prologue params are NULL");
  if (!(pro->norm_eps > 0.f) || !std::isfinite(pro->norm_eps))
    return fail(SA_ERR_PARAM, "norm_eps must be positive and finite");
  if (!(pro->rope_base > 0.f) || !std::isfinite(pro->rope_base))
    return fail(SA_ERR_PARAM, "rope_base must be positive and finite");
  if (r.qk != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "the producer step takes bf16 Q/K/V");
  if (r.empty) return ok();
  if (!q_gain || !k_gain || !q_out || !k_out) return fail(SA_ERR_NULL, "gain or output is NULL");
  if (!aligned(q_gain, 4) || !aligned(k_gain, 4)) return fail(SA_ERR_ALIGN, "gains must be 4-byte aligned");
  if (!aligned(q_out, 16) || !aligned(k_out, 16)) return fail(SA_ERR_ALIGN, "outputs must be 16-byte aligned");
  if ((s = check_ws(ws, ws_bytes, r)) != SA_OK) return s;
  sa::PoolArgs a = pool_args(r, in, ws, false);
  a.pro.on = true;
  a.pro.q_gain = q_gain;
  a.pro.k_gain = k_gain;
  a.pro.q_out = static_cast<uint16_t*>(q_out);
  a.pro.k_out = static_cast<uint16_t*>(k_out);
  a.pro.eps = pro->norm_eps;
  a.pro.base = pro->rope_base;
  a.pro.T = r.T;
  a.pro.Hg = r.Hg;
  a.pro.Wg = r.Wg;
  return hip_status(sa::launch_pool(a, (hipStream_t)stream), "producer kernel launch");
}

SA_API sa_status sa_dense_forward(const sa_shape* shape, float scale, const sa_inputs* in, void* o,
                                  float* lse, void* ws, size_t ws_bytes, void* stream) {
  Req r{};
  sa_status s;
  if ((s = check_shape_inputs(shape, in, &r, true)) != SA_OK) return s;
  if (!std::isfinite(scale)) return fail(SA_ERR_PARAM, "scale must be finite");
  r.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)r.D);
  r.tau = INFINITY;
  r.topk = 0;
  r.correction = 0;
  if (r.empty) return ok();
  if ((s = check_out(o, lse, nullptr)) != SA_OK) return s;
  if ((s = check_ws(ws, ws_bytes, r)) != SA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (r.v == SA_BF16) {
    if ((s = hip_status(sa::launch_pool(pool_args(r, in, ws, true), st), "regroup kernel launch")) !=
        SA_OK)
      return s;
  }
  return run_attn(r, in, o, lse, nullptr, ws, false, st);
}
