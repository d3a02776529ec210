/*
 * sa_route.h -- C ABI of the on-the-fly block-sparse self-attention library
 * for AMD Instinct MI355X (gfx950).  Library: libsa_route.so.
 *
 * Operation (Sol-Attn project page, nvlabs.github.io/Sana/Sol-Attn, section
 * "Abstract"; Sol-Engine README, section "Sol-Attention"): video-token
 * self-attention in which every query block is routed, by a query-dependent
 * threshold on a pooled score computed on chip, to the key blocks it attends
 * exactly; the skipped blocks are not dropped but enter through a cheap
 * correction; routing, sparse compute and correction share one online-softmax
 * pass.  The concrete reading implemented here, per (batch b, head h), with
 * block size beta = 64, Nb = ceil(N / 64), block J = tokens
 * [64J, min(64J + 64, N)) of size n_J, and s = scale (1/sqrt(D) by default):
 *
 *   pool     qbar_I, kbar_J, vbar_J = means over the tokens of each block
 *   route    p_IJ = s * qbar_I . kbar_J ;  keep_IJ = p_IJ >= max_J p_IJ - tau
 *            (or, with a fixed budget topk, the topk largest p_IJ of row I)
 *   exact    logits s * q_i . k_j for the tokens j of kept blocks
 *   correct  each skipped J acts as n_J copies of (kbar_J, vbar_J): logit
 *            s * q_i . kbar_J with weight n_J (only if correction != 0);
 *            with correction == 2 the value is instead the first-order one,
 *            vbar_J + (s / n_J) sum_j (qbar_I . (k_j - kbar_J)) v_j
 *   output   o_i = softmax-weighted sum of values over all those logits,
 *            lse_i = natural-log log-sum-exp of the weighted logits.
 *
 * tau = +INFINITY keeps every block: plain dense softmax attention.
 *
 * Conventions for every entry point:
 *  - Tensors are row-major and contiguous.  Q, K, V, O are [B, H, N, D];
 *    LSE is [B, H, N] float32; fp8 block scales are [B, H, Nb] float32;
 *    masks are [B, H, Nb, Nb] uint8 (0/1); kept counts are [B, H, Nb] int32.
 *  - Pointers to tensors and the workspace are DEVICE pointers, owned by the
 *    caller; shape/params/inputs structs are HOST pointers, read during the
 *    call only.  The library allocates no memory and keeps no per-call state.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work and return; they never synchronise.
 *  - All arguments are validated on the host before anything is enqueued.
 *    On any error the call returns a nonzero sa_status and enqueues nothing;
 *    sa_last_error() then describes the failure (per calling thread).  A
 *    failed kernel launch returns SA_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Outputs must not alias inputs or the workspace; they are fully
 *    overwritten.  Calls on different streams need distinct workspaces.
 *  - A call with B*H*N == 0 is valid, touches no pointer and returns SA_OK.
 *  - Results are bitwise deterministic for fixed inputs on a given device.
 *  - Supported: D in {64, 128}; block = 64; N <= SA_MAX_N; dtype pairs
 *    (qk, v) in {(F32, F32), (BF16, BF16), (FP8_E4M3, BF16)}.
 *  - Alignment: q, k, v, o and the workspace 16 bytes; lse, kept, scales 4.
 */
#ifndef SA_ROUTE_H
#define SA_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 4
#define SA_BLOCK 64
#define SA_MAX_NB 4096
#define SA_MAX_N (SA_BLOCK * SA_MAX_NB)

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is NULL */
  SA_ERR_SHAPE = 2,       /* bad B/H/N/D, N != T*Hg*Wg, N > SA_MAX_N, or B*H*Nb > 2^31 - 1 */
  SA_ERR_PARAM = 3,       /* block != 64, tau < 0 or NaN, topk < 0, bad correction flag, bad scale */
  SA_ERR_DTYPE = 4,       /* unsupported (qk_dtype, v_dtype) pair or scales given/missing */
  SA_ERR_ALIGN = 5,       /* pointer misaligned */
  SA_ERR_WORKSPACE = 6,   /* workspace smaller than sa_workspace_bytes() */
  SA_ERR_UNSUPPORTED = 7, /* valid request the library does not implement */
  SA_ERR_HIP = 8          /* a HIP runtime call or kernel launch failed */
} sa_status;

typedef enum sa_dtype {
  SA_F32 = 0,
  SA_BF16 = 1,
  SA_FP8_E4M3 = 2         /* OCP e4m3fn (max 448), with one fp32 scale per 64-token block */
} sa_dtype;

/* Q/K/V shape and the video token grid.  Tokens are in frame-major raster
 * order, token n = (t*Hg + y)*Wg + x; N must equal T*Hg*Wg.  Blocks are 64
 * consecutive tokens of this order (Sol-Engine README, "Sol-Attention":
 * the replaced operator is video-token self-attention). */
typedef struct sa_shape {
  int32_t B, H, N, D;
  int32_t T, Hg, Wg;
} sa_shape;

/* Routing parameters (Sol-Attn page, "Abstract": query-dependent threshold).
 * block: must be 64.  tau: threshold below the row maximum of the proxy, in
 * scaled-logit (natural log) units; tau >= 0, +INFINITY keeps every block.
 * correction: 1 = add the skipped-block correction (each skipped block as n_J
 * copies of its mean key and mean value), 0 = drop skipped blocks, 2 = the
 * first-order correction: PISA compensates non-critical blocks with a
 * first-order Taylor approximation (paper review of the Sol Video Inference
 * Engine, xllm-io blog, five acceleration techniques, item "Sparse
 * Attention").  Read here as the expansion of exp(s q_i . k_j) to first order
 * in the key's deviation d_j = k_j - kbar_J, coefficient taken at the query
 * block mean: a skipped block keeps the weight n_J exp(s q_i . kbar_J) and
 * takes the value vbar_J + (s / n_J) sum_j (qbar_I . d_j) v_j (fp8 keys:
 * dequantised).  The attention call (sa_forward, sa_forward_pooled) computes
 * these values, one D-vector per (query block, key block), for a slab of
 * heads at a time right before the attention over that slab, with this
 * params' scale; the workspace grows by one slab of values (see
 * sa_first_order_slab_heads: at most 8 GiB, or one head where a head needs
 * more).  Every dtype pair supports it.
 * scale: softmax scale s; <= 0 selects 1/sqrt(D); must be finite.
 * topk: 0 = threshold routing with tau; > 0 = fixed budget instead: every
 * query block keeps the min(topk, Nb) key blocks of largest proxy, equal
 * proxies in increasing block order, and tau is ignored (PISA at a fixed
 * sparsity, paper review of the Sol Video Inference Engine, xllm-io blog:
 * sparsity f corresponds to topk = ceil((1 - f) * Nb)).  topk < 0 is
 * SA_ERR_PARAM.
 * tile_t, tile_h, tile_w: 0, 0, 0 = blocks are 64 consecutive tokens of the
 * raster order.  Otherwise (each >= 1, product 64) blocks are formed over the
 * tokens in 3-D tile order: first every full tile_t x tile_h x tile_w tile of
 * the grid, tiles in raster order of their tile coordinates and tokens inside
 * a tile in (t, y, x) order, then the tokens no full tile covers, in raster
 * order; so every full tile is one block.  Masks, kept counts and the
 * means index these blocks; O and LSE stay in the caller's token order.
 * Needs bf16 or fp32 Q/K (fp8 block scales belong to raster blocks:
 * SA_ERR_UNSUPPORTED); the workspace grows by a copy of K in tile order.
 * Reading of video-token blocks on the grid (Sol-Engine README,
 * "Sol-Attention"). */
typedef struct sa_params {
  int32_t block;
  float tau;
  int32_t correction;
  float scale;
  int32_t topk;
  int32_t tile_t, tile_h, tile_w;
} sa_params;

/* Input tensors.  q_scale/k_scale: [B, H, Nb] fp32 block scales, required
 * iff qk_dtype == SA_FP8_E4M3 (element value = code * scale of its block),
 * otherwise must be NULL.  qk_dtype / v_dtype are sa_dtype values. */
typedef struct sa_inputs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_scale;
  const float* k_scale;
  int32_t qk_dtype;
  int32_t v_dtype;
} sa_inputs;

/* Parameters of the fused Q/K producer step (sa_qk_prologue). */
typedef struct sa_prologue {
  float norm_eps;   /* RMS-norm epsilon, > 0 */
  float rope_base;  /* rotary frequency base, > 0 (10000 in most models) */
} sa_prologue;

/* ABI version of the loaded library (SA_ABI_VERSION it was built with). */
int32_t sa_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* sa_status_string(sa_status s);

/* Detail of the last failed call made by this thread (static per thread;
 * empty string if none). */
const char* sa_last_error(void);

/* Status of the last call made by this thread (SA_OK after a successful
 * call): the reason when a size query below returns 0. */
sa_status sa_last_status(void);

/* Workspace bytes that sa_pool / sa_route / sa_forward / sa_forward_pooled
 * need for this shape, dtypes and params (block means in fp32; for bf16 V the
 * key means in two bf16 halves, the bf16 value means and V regrouped per
 * 64-key block; 256 bytes of counters of the attention kernel's workgroup
 * schedule; K in tile order with a 3-D tile order; one slab of first-order
 * values with correction == 2).  Returns 0 if the arguments are invalid.
 * Pass params = NULL for the default params. */
size_t sa_workspace_bytes(const sa_shape* shape, const sa_params* params, const sa_inputs* in);

/* Step "pool" (the pooled score's operands): writes qbar, kbar, vbar (fp32
 * means over each block's actual n_J tokens; fp8 inputs are dequantised with
 * their block scale), the bf16 copies of the means and the regrouped V used
 * by the attention kernels into the workspace. */
sa_status sa_pool(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                  void* ws, size_t ws_bytes, void* stream);

/* Steps "pool" + "route", standalone, for inspection and tests: writes the
 * 0/1 keep mask [B, H, Nb, Nb] (mask[b][h][I][J] = 1 iff query block I keeps
 * key block J) and, if kept != NULL, the kept count per query block
 * [B, H, Nb].  Uses the same device routine, in the same float32 order, as
 * sa_forward, so the two agree bit for bit. */
sa_status sa_route(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                   uint8_t* mask, int32_t* kept, void* ws, size_t ws_bytes, void* stream);

/* The fused path: pool, then one kernel that per query block computes the
 * proxy row on chip (never written out), thresholds it, folds the correction
 * of the skipped blocks into the running softmax max/sum, and runs exact
 * flash attention over the kept blocks.  Writes O ([B, H, N, D], dtype =
 * v_dtype) and LSE ([B, H, N] fp32, natural log, including correction mass);
 * kept (optional, [B, H, Nb] int32) receives each query block's kept count. */
sa_status sa_forward(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                     void* o, float* lse, int32_t* kept, void* ws, size_t ws_bytes, void* stream);

/* sa_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same pool and attention kernels, with the workspace in a static device
 * array of SA_NOALLOC_SCRATCH_BYTES (256 MiB) inside the library instead of
 * a caller buffer.  Each GPU the library runs on holds its own array until
 * the process ends; its address is looked up on the first call on a device.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  The caller still passes the inputs and outputs, as for
 * sa_forward.  A call whose workspace (sa_workspace_bytes) exceeds the array
 * returns SA_ERR_WORKSPACE and enqueues nothing.  Every call on a GPU shares
 * that GPU's array and leaves its contents behind; each call rewrites all it
 * reads.  Calls that overlap on one GPU (different streams or threads
 * without ordering between them) race on the array: serialise them. */
#define SA_NOALLOC_SCRATCH_BYTES (256u << 20)
sa_status sa_forward_noalloc(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                             void* o, float* lse, int32_t* kept, void* stream);

/* sa_forward without the pool step: the workspace must already hold the
 * output of sa_pool for the same inputs, shape and params. */
sa_status sa_forward_pooled(const sa_shape* shape, const sa_params* params, const sa_inputs* in,
                            void* o, float* lse, int32_t* kept, void* ws, size_t ws_bytes,
                            void* stream);

/* Fused Q/K producer step in place of sa_pool (the paper review of the Sol
 * Video Inference Engine, xllm-io blog, lists fused RoPE + norm and fused
 * QK + RoPE among the fusions in front of attention).  in->q and in->k hold
 * the raw per-head Q/K projections [B, H, N, D] (bf16), in->v the values
 * (bf16).  Every token row of Q and of K is
 *   RMS-normalised over its D features: x / sqrt(mean(x^2) + norm_eps),
 *   scaled by the gain (q_gain / k_gain: [D] fp32, shared by the heads),
 *   rotated pairwise by its grid position: feature pairs (2j, 2j+1) form
 *   three consecutive groups -- D - 4*(D/6) features for the frame index t,
 *   2*(D/6) for the row y, 2*(D/6) for the column x -- and pair j of a group
 *   of d_a features turns by pos_a * rope_base^(-2j/d_a) radians,
 *   rounded to bf16 and written to q_out / k_out ([B, H, N, D] bf16, token
 *   order; they may be in->q / in->k themselves, in place).
 * The workspace then holds exactly what sa_pool would compute from q_out,
 * k_out and v (block means over the blocks that params selects, the bf16
 * copies, V regrouped, K in tile order), so sa_forward_pooled with inputs
 * {q_out, k_out, v} and the same params completes the attention (with
 * correction == 2 that call also computes the first-order values, from the
 * produced Q/K and its own scale).  params is used for its block order and
 * workspace layout only.  Only bf16 Q/K/V (SA_ERR_UNSUPPORTED otherwise);
 * gains 4-byte aligned, outputs 16-byte aligned. */
sa_status sa_qk_prologue(const sa_shape* shape, const sa_params* params, const sa_prologue* pro,
                         const sa_inputs* in, const float* q_gain, const float* k_gain, void* q_out,
                         void* k_out, void* ws, size_t ws_bytes, void* stream);

/* Heads per slab of the first-order correction (params->correction == 2):
 * sa_forward / sa_forward_pooled compute the first-order values of this many
 * heads at a time, each slab right before the attention over it, and the
 * workspace holds one slab.  The slabs are the fewest of equal size (up to
 * one head) whose values fit in 8 GiB each, with Nb*Nbp*D bf16 values per
 * head (Nb*Nb*D fp32 for fp32 inputs), or one head per slab where one head
 * needs more.  This bounds the first-order workspace at 8 GiB, or one head.
 * Returns 0 on invalid arguments or B*H == 0. */
int64_t sa_first_order_slab_heads(const sa_shape* shape, const sa_inputs* in);

/* Fixed budget for a sparsity f (the fraction of the Nb = ceil(N / 64) key
 * blocks a query block skips; PISA runs at a fixed sparsity, paper review of
 * the Sol Video Inference Engine, xllm-io blog): topk = ceil((1 - f) * Nb),
 * at least 1 and at most Nb, for sa_params.topk.  A product within 1e-9 of
 * an integer counts as that integer.  Returns 0 (SA_ERR_PARAM in
 * sa_last_status) unless N >= 1 and 0 <= f < 1. */
int32_t sa_budget_blocks(int32_t N, double sparsity);

/* Workspace bytes for sa_dense_forward (0 on invalid arguments). */
size_t sa_dense_workspace_bytes(const sa_shape* shape, const sa_inputs* in);

/* Dense bidirectional softmax attention, the "Dense" baseline of the Sol-Attn
 * page and the tau = +INFINITY limit of sa_forward: O and LSE as above.
 * scale <= 0 selects 1/sqrt(D).  For bf16 V the workspace receives V
 * regrouped per 64-key block; for fp32 it may be NULL (size 0). */
sa_status sa_dense_forward(const sa_shape* shape, float scale, const sa_inputs* in,
                           void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_ROUTE_H */
