"""Plain CPU oracle for on-the-fly block-sparse self-attention (Sol-Attn style).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library and imports nothing from it.

What it computes
----------------
The Sol-Attn project page ("Sol-Attn: Accelerating Video Generation Inference
via On-the-Fly Attention Sparsification", nvlabs.github.io/Sana/Sol-Attn,
section "Abstract") describes one online-softmax pass that (i) routes each
query block to key blocks by a query-dependent threshold on a pooled score,
(ii) computes exact attention over the selected blocks and (iii) adds an
approximate correction for the long-tail mass of the skipped blocks by reusing
below-threshold score columns.  The Sol-Engine README (raw README of
NVlabs/Sana, branch sol-engine, section "Sol-Attention") adds that the
replaced operator is video-token self-attention computed only on the most
relevant key blocks, plus a light-weight compensating operation.

The pages give no formula, so this module fixes the plainest concrete reading
(every reading is listed in the design notes of the repository):

* tokens are split into blocks of ``block`` consecutive tokens; block J holds
  tokens [block*J, min(block*J + block, N)) and n_J is its actual size;
* the pooled score ("proxy") is p_IJ = s * mean(q over I) . mean(k over J),
  with s the softmax scale (1/sqrt(D) unless given);
* block J is kept for query block I iff p_IJ >= max_J' p_IJ' - tau
  (inclusive; tau = +inf keeps every block);
* each skipped block J is modelled as n_J copies of its mean key and mean
  value: row i sees the correction logit c_iJ = s * q_i . mean(k over J)
  with multiplicity n_J -- c_iJ is the (i, J) entry of s * Q_I Kbar^T, the
  "score column" of block J;
* the output is the softmax over the union of exact logits (kept blocks) and
  correction logits (skipped blocks, if correction is on), with natural-log
  LSE lse_i = M_i + ln Z_i;
* optionally (correction = 2) the skipped blocks are modelled to first order
  instead: PISA, as the paper review of the Sol Video Inference Engine
  (xllm-io blog, five acceleration techniques, item "Sparse Attention")
  describes it, computes critical blocks exactly and compensates the others
  with a first-order Taylor approximation.  With k_j = kbar_J + d_j and q_i = qbar_I + e_i, the exact
  weight exp(s q_i . k_j) is taken as exp(c_iJ) * (1 + s qbar_I . d_j): the
  factor exp(c_iJ) keeps the per-row score column exactly, the bracket is the
  first-order term in the key deviation, and the product term s e_i . d_j,
  second order in the deviations from the block means, is dropped (with q_i in
  place of qbar_I the first-order term would cost as much as the exact
  block).  Because the d_j of a block sum to zero, the block's weight is still
  n_J exp(c_iJ) and only its value changes, to
  vbar_J + (s / n_J) sum_j (qbar_I . d_j) v_j, one vector per (I, J);
* alternatively (route_topk) a fixed budget: each query block keeps the topk
  key blocks of largest proxy, equal proxies in increasing block order --
  the paper review of the Sol Video Inference Engine (xllm-io blog) runs
  PISA at block size 64 and a fixed sparsity rather than a threshold;
* optionally the tokens are first put in 3-D tile order (tile_order): blocks
  are then cubes of the video token grid rather than raster segments.

It is evaluated here as the two-pass definition above in float64, not as an
online softmax: first every logit of a row, then its max, then the sums.
Each function below says which step it is.

Pinned by tests/test_oracle_pins.py, tests/test_oracle_topk.py and
tests/test_oracle_tiles.py (closed forms of hand-derived cases, pure-Python
brute force, library special cases, invariants) and, for the first-order
model, tests/test_oracle_taylor.py (per-key brute force, O(t^2) convergence
to dense attention, reductions to the mean copies, invariants);
tests/test_oracle_mutants.py and the mutants in test_oracle_taylor.py check
that planted mistakes fail those pins.  Parity unpinned: none.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "block_ranges",
    "block_means",
    "default_scale",
    "proxy_scores",
    "route",
    "route_topk",
    "tile_order",
    "first_order_value",
    "attend_rows",
    "forward_head",
    "forward",
    "dense_head",
]


def default_scale(D: int, scale: float | None = None) -> float:
    """Softmax scale: 1/sqrt(D) unless an explicit positive scale is given.

    The usual scaled-dot-product attention convention; the Sol-Engine README
    (section "Sol-Attention") presents the sparse kernel as a drop-in for the
    model's dense self-attention, which uses this scale.
    """
    if scale is not None and scale > 0:
        return float(scale)
    return 1.0 / math.sqrt(D)


def block_ranges(N: int, block: int) -> list[tuple[int, int]]:
    """Token ranges of the blocks: 64 consecutive tokens each (the last one ragged).

    Blocks follow the given token order (frame-major raster of the video token
    grid); no 3-D tiling or reordering is applied.
    """
    if block <= 0:
        raise ValueError("block must be positive")
    return [(s, min(s + block, N)) for s in range(0, N, block)]


def tile_order(T: int, Hg: int, Wg: int, tile) -> np.ndarray:
    """Token order that makes blocks 3-D tiles of the video token grid.

    Position -> token index (token n = (t*Hg + y)*Wg + x in the frame-major
    raster).  First every full tile of tile = (tt, th, tw) tokens, tiles in
    raster order of their (frame, row, column) tile coordinates and tokens
    within a tile in (t, y, x) raster order; then every token that no full
    tile covers, in the raster order.  With tt*th*tw equal to the block size
    each full tile is exactly one block.  Reading of "3-D tile block ordering
    from the grid": the Sol-Engine README (section "Sol-Attention") replaces
    video-token self-attention, whose tokens live on this grid.
    """
    tt, th, tw = (int(x) for x in tile)
    if min(tt, th, tw) < 1:
        raise ValueError("tile dimensions must be positive")
    nz, ny, nx = T // tt, Hg // th, Wg // tw
    order = []
    for fz in range(nz):
        for fy in range(ny):
            for fx in range(nx):
                for dz in range(tt):
                    for dy in range(th):
                        for dx in range(tw):
                            t, y, x = fz * tt + dz, fy * th + dy, fx * tw + dx
                            order.append((t * Hg + y) * Wg + x)
    for t in range(T):
        for y in range(Hg):
            for x in range(Wg):
                if t >= nz * tt or y >= ny * th or x >= nx * tw:
                    order.append((t * Hg + y) * Wg + x)
    return np.array(order, dtype=np.int64)


def block_means(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of each block's rows over the block's actual token count.

    Step "pooled score" of the Sol-Attn Abstract, read as block means.
    x: [N, D] float64 -> [Nb, D] float64.
    """
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[0]
    out = np.empty((len(block_ranges(N, block)), x.shape[1]), dtype=np.float64)
    for J, (s, e) in enumerate(block_ranges(N, block)):
        out[J] = x[s:e].sum(axis=0) / (e - s)
    return out


def proxy_scores(q: np.ndarray, k: np.ndarray, block: int, scale: float | None = None) -> np.ndarray:
    """Proxy p[I, J] = s * qbar_I . kbar_J for every query block I and key block J.

    The Abstract's pooled score; the kernel evaluates one row of it on chip and
    never writes the map out.  Here the whole [Nb, Nb] map is formed on the CPU.
    """
    s = default_scale(q.shape[1], scale)
    qb = block_means(q, block)
    kb = block_means(k, block)
    return s * (qb @ kb.T)


def route(q: np.ndarray, k: np.ndarray, block: int, tau: float, scale: float | None = None):
    """Query-dependent threshold routing (Sol-Attn Abstract).

    keep[I, J] = p[I, J] >= max_J' p[I, J'] - tau   (inclusive).
    Returns (keep bool [Nb, Nb], p [Nb, Nb], rowmax [Nb]).
    """
    tau = float(tau)
    if math.isnan(tau) or tau < 0:
        raise ValueError("tau must be >= 0 (or +inf)")
    p = proxy_scores(q, k, block, scale)
    m = p.max(axis=1)
    keep = p >= (m - tau)[:, None]
    return keep, p, m


def route_topk(q: np.ndarray, k: np.ndarray, block: int, topk: int, scale: float | None = None):
    """Fixed-budget routing: keep the min(topk, Nb) key blocks with the
    largest proxy in each query block's row; equal proxies are taken in
    increasing key-block order.

    The paper review of the Sol Video Inference Engine (xllm-io blog,
    technique list, item "Sparse Attention", and the LTX-2.3 pipeline
    settings) runs PISA with block size 64 at a fixed sparsity of 0.9, i.e. a
    per-query-block budget of key blocks rather than a threshold; the score
    ranked is the same pooled proxy as in route().
    Returns (keep bool [Nb, Nb], p [Nb, Nb], pk [Nb]) with pk[I] the proxy of
    the last block kept in row I (the k-th largest).
    """
    topk = int(topk)
    if topk < 1:
        raise ValueError("topk must be >= 1")
    p = proxy_scores(q, k, block, scale)
    nb = p.shape[0]
    kk = min(topk, nb)
    keep = np.zeros((nb, nb), dtype=bool)
    pk = np.empty(nb)
    for I in range(nb):
        # primary key: proxy, descending; secondary: block index, ascending
        order = np.lexsort((np.arange(nb), -p[I]))
        keep[I, order[:kk]] = True
        pk[I] = p[I, order[kk - 1]]
    return keep, p, pk


def first_order_value(qbar: np.ndarray, kJ: np.ndarray, vJ: np.ndarray, s: float) -> np.ndarray:
    """Value of a skipped key block under the first-order model (module
    docstring): vbar_J + (s / n_J) sum_j (qbar_I . (k_j - kbar_J)) v_j.

    qbar: [D] mean of the query block; kJ: [n_J, D], vJ: [n_J, Dv] the block's
    keys and values; s: the softmax scale.
    """
    kJ = np.asarray(kJ, dtype=np.float64)
    vJ = np.asarray(vJ, dtype=np.float64)
    d = kJ - kJ.mean(axis=0)                  # key deviations from the block mean
    return vJ.mean(axis=0) + (s * (d @ np.asarray(qbar, dtype=np.float64))) @ vJ / kJ.shape[0]


def attend_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, keep_row: np.ndarray,
                block: int, correction, scale: float | None = None):
    """Output and LSE of the rows of one query block, given its keep row.

    q_rows: [n_I, D], all rows of the query block; k: [N, D]; v: [N, Dv];
    keep_row: bool [Nb].  correction: 0 / False none, 1 / True the mean
    copies, 2 the first-order model (module docstring).
    Two passes over all logits of each row (exact logits of kept blocks, then
    the correction logits of skipped blocks with multiplicity n_J), max, sums.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = default_scale(q_rows.shape[1], scale)
    N = k.shape[0]
    ranges = block_ranges(N, block)
    kept = [J for J in range(len(ranges)) if keep_row[J]]
    skipped = [J for J in range(len(ranges)) if not keep_row[J]]

    # exact logits s_ij over the tokens of the kept blocks
    idx = np.concatenate([np.arange(*ranges[J]) for J in kept]) if kept else np.zeros(0, dtype=np.int64)
    logits = s * (q_rows @ k[idx].T)                       # [n_I, n_kept_tokens]
    weights_mult = np.ones(idx.shape[0])
    values = v[idx]

    if correction and skipped:
        kbar = np.stack([k[slice(*ranges[J])].mean(axis=0) for J in skipped])
        vbar = np.stack([v[slice(*ranges[J])].mean(axis=0) for J in skipped])
        nJ = np.array([ranges[J][1] - ranges[J][0] for J in skipped], dtype=np.float64)
        if correction == 2:
            qbar = q_rows.mean(axis=0)
            for t, J in enumerate(skipped):
                vbar[t] = first_order_value(qbar, k[slice(*ranges[J])], v[slice(*ranges[J])], s)
        c = s * (q_rows @ kbar.T)                          # score columns of skipped blocks
        logits = np.concatenate([logits, c], axis=1)
        weights_mult = np.concatenate([weights_mult, nJ])
        values = np.concatenate([values, vbar], axis=0)

    M = logits.max(axis=1, keepdims=True)
    w = weights_mult[None, :] * np.exp(logits - M)         # n_J copies -> weight n_J
    Z = w.sum(axis=1, keepdims=True)
    o = (w @ values) / Z
    lse = M[:, 0] + np.log(Z[:, 0])
    return o, lse


def forward_head(q, k, v, block: int = 64, tau: float = math.inf, correction=True,
                 scale: float | None = None, keep: np.ndarray | None = None,
                 qblocks=None, topk: int | None = None, order=None):
    """Sparse attention of one (batch, head): returns (o [N, Dv], lse [N], keep).

    keep: optional externally supplied [Nb, Nb] mask replacing the routing
    (used to evaluate the definition on a mask that differs from this oracle's
    only inside the near-threshold band).  qblocks: optional iterable of query
    block indices; rows of other blocks are left as NaN.  topk: route with the
    fixed budget of route_topk() instead of the threshold tau.  order:
    optional position -> token permutation (tile_order()); blocks are then
    formed over the permuted tokens, keep and qblocks index those blocks, and
    o / lse are returned in the original token order.
    """
    if order is not None:
        order = np.asarray(order)
        o_p, lse_p, keep = forward_head(np.asarray(q)[order], np.asarray(k)[order], np.asarray(v)[order],
                                        block, tau, correction, scale, keep, qblocks, topk)
        o = np.empty_like(o_p)
        lse = np.empty_like(lse_p)
        o[order] = o_p
        lse[order] = lse_p
        return o, lse, keep
    q = np.asarray(q, dtype=np.float64)
    N = q.shape[0]
    if keep is None:
        if topk:
            keep, _, _ = route_topk(q, k, block, topk, scale)
        else:
            keep, _, _ = route(q, k, block, tau, scale)
    ranges = block_ranges(N, block)
    o = np.full((N, np.asarray(v).shape[1]), np.nan)
    lse = np.full(N, np.nan)
    for I in (range(len(ranges)) if qblocks is None else qblocks):
        a, b = ranges[I]
        o[a:b], lse[a:b] = attend_rows(q[a:b], k, v, keep[I], block, correction, scale)
    return o, lse, keep


def forward(q, k, v, block: int = 64, tau: float = math.inf, correction=True,
            scale: float | None = None, topk: int | None = None, order=None):
    """[B, H, N, D] batched form of forward_head; every (b, h) routes independently."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, _ = q.shape
    o = np.empty(q.shape[:3] + (np.asarray(v).shape[3],))
    lse = np.empty((B, H, N))
    keep = np.empty((B, H, (N + block - 1) // block, (N + block - 1) // block), dtype=bool)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], keep[b, h] = forward_head(q[b, h], k[b, h], v[b, h], block, tau,
                                                          correction, scale, topk=topk, order=order)
    return o, lse, keep


def dense_head(q, k, v, scale: float | None = None, rows=None):
    """Dense bidirectional softmax attention of one head (the tau = inf limit).

    The baseline every speedup on the Sol-Attn page is quoted against
    (labelled "Dense").  rows: optional index array of query rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = default_scale(q.shape[1], scale)
    qr = q if rows is None else q[rows]
    logits = s * (qr @ k.T)
    M = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - M)
    Z = w.sum(axis=1, keepdims=True)
    return (w @ v) / Z, M[:, 0] + np.log(Z[:, 0])
