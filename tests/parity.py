"""Parity helpers: HIP results against the CPU oracle on the same seeded inputs.

Tolerances (fixed by the method's stated bars):
* float32 path: row-normwise relative error of O <= 1e-5
  (max_i |o_i - ref_i|_inf / |ref_i|_inf) and |LSE - ref| <= 1e-5 * max(1, |ref|);
* bf16 path: max |O - ref| <= 2e-2 and mean |O - ref| <= 2e-3 against the
  float64 oracle on the same bf16-rounded inputs;
* fp8 Q/K path: max |O - ref| <= 4e-2 against the oracle on the dequantised
  inputs;
* masks: bit-exact except blocks whose float64 proxy lies within 1e-3 of the
  threshold (those are counted); outputs are then compared with the oracle
  evaluated on the GPU's mask.
LSE of the bf16/fp8 paths has no stated bar; the bound used (1e-2 absolute)
is derived next to TOL below from the bf16 rounding of P.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import attention as orc

BAND = 1e-3
# O tolerances are the stated bars (fp32: row-normwise relative 1e-5; bf16: max
# abs 2e-2, mean abs 2e-3; fp8: max abs 4e-2).  LSE has no stated bar; ours is
# derived from the arithmetic: every logit is exact up to float32 rounding
# (bf16 or fp8 products accumulated in float32; the correction logits take
# the key means in two bf16 halves, about 16 significant bits, so
# s*q.kbar is off by about 2^-17 of s*|q||kbar|), and the row sum is taken
# over weights rounded to bf16 (relative 2^-8 at most each), so the LSE is off
# by at most about 2^-8 = 4e-3: 1e-2 for bf16 and fp8.
TOL = {
    "f32": dict(row_rel=1e-5, lse_rel=1e-5),
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, lse_abs=1e-2),
    "fp8": dict(max_abs=4e-2, lse_abs=1e-2),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_map(fn, items, workers: int = 8):
    """fn over items in a thread pool, for oracle work on many heads.  BLAS
    runs one thread per call meanwhile: concurrent multi-threaded BLAS calls
    from several threads have returned wrong products with this numpy's
    OpenBLAS."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def to_gpu(inp):
    dev = torch.device("cuda:0")
    g = lambda t: None if t is None else t.to(dev).contiguous()  # noqa: E731
    return g(inp.q), g(inp.k), g(inp.v), g(inp.q_scale), g(inp.k_scale)


def grid_of(wl):
    return (wl.T, wl.Hg, wl.Wg)


def _head(inp, b, h, order):
    q, k, v = inp.head64(b, h)
    if order is not None:
        q, k, v = q[order], k[order], v[order]
    return q, k, v


def mask_check(inp, b, h, gpu_mask: np.ndarray, tau: float, scale=None, order=None):
    """Compare the GPU keep mask of one head with the float64 routing.

    Returns (keep_for_oracle, n_band, n_flipped_in_band); asserts that no block
    outside the near-threshold band differs.  order: position -> token map of
    the blocks (3-D tile order), None for the raster order."""
    q, k, _ = _head(inp, b, h, order)
    keep, p, m = orc.route(q, k, inp.wl.block, tau, scale)
    gm = gpu_mask.astype(bool)
    if math.isinf(tau):
        band = np.zeros_like(keep)
    else:
        band = np.abs(p - (m - tau)[:, None]) < BAND
    diff = gm != keep
    outside = diff & ~band
    assert not outside.any(), (
        f"head ({b},{h}): {int(outside.sum())} mask entries differ outside the {BAND} band, "
        f"first at {np.argwhere(outside)[0].tolist()}")
    return gm, int(band.sum()), int((diff & band).sum())


def mask_check_topk(inp, b, h, gpu_mask: np.ndarray, topk: int, scale=None, order=None):
    """Fixed-budget routing: the GPU keeps exactly min(topk, Nb) blocks per
    query block, and differs from the float64 selection only for blocks whose
    proxy lies within the band of the row's k-th largest proxy."""
    q, k, _ = _head(inp, b, h, order)
    keep, p, pk = orc.route_topk(q, k, inp.wl.block, topk, scale)
    gm = gpu_mask.astype(bool)
    nb = keep.shape[0]
    assert (gm.sum(axis=1) == min(topk, nb)).all(), "kept count differs from the budget"
    band = np.abs(p - pk[:, None]) < BAND
    diff = gm != keep
    outside = diff & ~band
    assert not outside.any(), (
        f"head ({b},{h}): {int(outside.sum())} mask entries differ outside the {BAND} band, "
        f"first at {np.argwhere(outside)[0].tolist()}")
    return gm, int(band.sum()), int((diff & band).sum())


def output_check(inp, b, h, o_gpu: torch.Tensor, lse_gpu: torch.Tensor, keep: np.ndarray, tau: float,
                 correction: bool, qblocks=None, scale=None, dense=False, order=None):
    """Oracle output for the given query blocks of head (b, h) against the GPU's.

    order: position -> token map (3-D tile order); qblocks and keep then index
    blocks of positions, and the rows compared are the tokens they hold."""
    wl = inp.wl
    q, k, v = inp.head64(b, h)
    N = q.shape[0]
    ranges = orc.block_ranges(N, wl.block)
    qblocks = list(range(len(ranges))) if qblocks is None else sorted(set(qblocks))
    rows = np.concatenate([np.arange(*ranges[I]) for I in qblocks])
    if order is not None:
        rows = np.asarray(order)[rows]
    if dense:
        o_ref, lse_ref = orc.dense_head(q, k, v, scale, rows=rows)
    else:
        o_full, lse_full, _ = orc.forward_head(q, k, v, wl.block, tau, correction, scale, keep=keep,
                                               qblocks=qblocks, order=order)
        o_ref, lse_ref = o_full[rows], lse_full[rows]
    o = o_gpu[b, h].float().cpu().numpy().astype(np.float64)[rows]
    lse = lse_gpu[b, h].cpu().numpy().astype(np.float64)[rows]
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "non-finite GPU output"
    err = np.abs(o - o_ref)
    lerr = np.abs(lse - lse_ref)
    t = TOL[wl.dtype]
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_abs=float(lerr.max()))
    if wl.dtype == "f32":
        row_rel = (err.max(axis=1) / np.maximum(np.abs(o_ref).max(axis=1), 1e-30)).max()
        stats["row_rel"] = float(row_rel)
        assert row_rel <= t["row_rel"], stats
        assert (lerr <= t["lse_rel"] * np.maximum(1.0, np.abs(lse_ref))).all(), stats
    else:
        assert stats["max_abs"] <= t["max_abs"], stats
        if "mean_abs" in t:
            assert stats["mean_abs"] <= t["mean_abs"], stats
        assert stats["lse_abs"] <= t["lse_abs"], stats
    return stats
