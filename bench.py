#!/usr/bin/env python3
"""Benchmark of the on-the-fly block-sparse attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p] [--tau 2]
                    [--budgets 0.9,0.8] [--configs 720p:4,...] [--no-cpu-baseline]

A step is one sa_forward call (pool kernel + fused route/correct/attend
kernel) over the whole workload, inputs resident in HBM.  Prints one JSON
line on stdout; diagnostics go to stderr.

value = computed-block TFLOP/s: sum over kept (query block, key block) pairs
of 4*D*n_I*n_J, divided by the wall time of one call.  The roofline object
covers the fused kernel, timed with HIP events recorded on the stream the
library launches on, around each launch inside the timed region.  The
cpu_baseline leg times the float64 CPU oracle on whole heads of the same
workload (routing and attention of every query block of head (0, 0)) and
reports it in the same unit.
The fixed_budget list times the same call with routing by a fixed number of
key blocks per query block (sparsity 0.9 and 0.8 by default) instead of tau;
the tile_order list times it with blocks formed over 3-D tiles of the token
grid (4x4x4 and 1x8x8 by default); fused_producer times sa_qk_prologue (norm
+ rotary + pool of the Q/K projections) in place of the pool; first_order
times the call with the first-order correction of the skipped blocks
(correction = 2: the attention call computes the per-pair values a slab of
heads at a time and the fused kernel reads them) and its error against dense
attention.  The configs list
repeats the call (a few steps each) at the other workloads: 720p at tau 4
and 8, 480p, 1080p and the 720p CFG batch with fp8 Q/K, each with its dense
call, density, and -- from the CPU leg -- the near-threshold and flipped
block counts of every head.

gemm_reference times a plain 16384^3 bf16 GEMM through torch.matmul (the
vendor's GEMM library) in the same run: the matrix-core rate this GPU
sustains for dense bf16 work, next to the published peak the roofline uses.

Pool bandwidth is quoted on the pass's algorithmic bytes (Q, K and V read
once plus the three float32 mean tensors written, and the fp8 block scales),
with this library's own layout bytes (bf16 key/value means and V regrouped
per block, written for the attention kernel) beside them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_attention_route_amd import api, synth  # noqa: E402

METRIC = "sparse-attn ms/call + computed-block TFLOPS (% MFMA peak), 720p video DiT shape"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_kernel_traffic.json")
KERNEL_SOURCES = ["attn_mfma.hip", "sa_device.h", "sa_layout.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed: the hash
    identifies the code the counters were taken on, not its comments."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_attention_route_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def union_inflation(mask: np.ndarray, group: int = 4) -> float:
    """Tiles a workgroup of `group` adjacent query blocks streams (the union of
    their kept lists) over the mean kept count, averaged over the launch."""
    bh, nb, _ = mask.shape
    pad = (-nb) % group
    m = np.concatenate([mask, np.zeros((bh, pad, nb), dtype=mask.dtype)], axis=1) if pad else mask
    groups = m.reshape(bh, -1, group, nb).astype(bool)
    union = groups.any(axis=2).sum()
    return float(union * group) / max(float(mask.astype(bool).sum()), 1.0)


def computed_block_flops(mask: np.ndarray, N: int, D: int) -> float:
    """sum over kept (I, J) of 4*D*n_I*n_J for a [BH, Nb, Nb] 0/1 mask."""
    Nb = mask.shape[-1]
    n = np.full(Nb, 64.0)
    n[-1] = N - 64 * (Nb - 1)
    per_row = (mask.astype(np.float64) * n[None, None, :]).sum(axis=-1)   # [BH, Nb]
    return float(4.0 * D * (per_row * n[None, :]).sum())


def correction_flops(mask: np.ndarray, N: int, D: int) -> float:
    """4*D*n_I per skipped (I, J) pair (score column and value of the correction)."""
    Nb = mask.shape[-1]
    n = np.full(Nb, 64.0)
    n[-1] = N - 64 * (Nb - 1)
    skipped = (1 - mask.astype(np.float64)).sum(axis=-1)
    return float(4.0 * D * (skipped * n[None, :]).sum())


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(inp, wl, tau, o_gpu, heads: int = 1):
    """Time the float64 oracle on whole heads of the workload: the routing of
    every query block and the attention of every query block of heads
    (0, 0), (0, 1), ...  One process; numpy's BLAS uses its thread pool."""
    from oracle import attention as orc  # test infrastructure: cpu_baseline leg only
    ranges = orc.block_ranges(wl.N, wl.block)
    n = np.array([e - s for s, e in ranges], dtype=np.float64)
    flops, t_route, t_attend, maxerr, nband = 0.0, 0.0, 0.0, 0.0, 0
    done = []
    for hh in range(heads):
        b, h = divmod(hh, wl.H)
        q, k, v = inp.head64(b, h)
        t0 = time.perf_counter()
        keep, p, m = orc.route(q, k, wl.block, tau)
        t_route += time.perf_counter() - t0
        o_g = o_gpu[b, h].float().cpu().numpy()
        t1 = time.perf_counter()
        for I, (a0, a1) in enumerate(ranges):
            o_ref, _ = orc.attend_rows(q[a0:a1], k, v, keep[I], wl.block, wl.correction)
            maxerr = max(maxerr, float(np.abs(o_ref - o_g[a0:a1]).max()))
            flops += 4.0 * wl.D * n[I] * float((keep[I] * n).sum())
        t_attend += time.perf_counter() - t1
        nband += int((np.abs(p - (m - tau)[:, None]) < 1e-3).sum()) if math.isfinite(tau) else 0
        done.append((b, h))
    elapsed = t_route + t_attend
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": _blas_threads(),
        "cores_kind": "BLAS threads of one numpy process",
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle, {len(done)} whole head(s) {done} of {wl.name}: routing of all "
                   f"{len(ranges)} query blocks ({t_route:.2f} s) and attention of all {len(ranges)} query "
                   f"blocks ({t_attend:.2f} s); computed-block FLOP of the sample / time"),
        "sample_s": elapsed,
        "sample_max_abs_err_vs_gpu": maxerr,
        # the whole call at the sample's rate per head: an extrapolation, not a measurement
        "extrapolated_call_s": elapsed / len(done) * wl.B * wl.H,
        "near_threshold_blocks_sampled_heads": nband,
    }


def route_band_counts(inp, wl, tau, gpu_mask: np.ndarray) -> dict:
    """The float64 routing of every head against the GPU's keep mask: blocks
    whose proxy lies within 1e-3 of the threshold, how many of those the GPU
    decided the other way, and differences outside that band (must be 0).
    Runs in the cpu_baseline leg (it is the oracle's routing)."""
    from oracle import attention as orc  # test infrastructure: cpu_baseline leg only
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    def one(bh):
        b, h = divmod(bh, wl.H)
        q, k, _ = inp.head64(b, h)
        keep, p, m = orc.route(q, k, wl.block, tau)
        band = np.abs(p - (m - tau)[:, None]) < 1e-3
        diff = gpu_mask[bh].astype(bool) != keep
        return int(band.sum()), int((diff & band).sum()), int((diff & ~band).sum())

    t0 = time.perf_counter()
    # one BLAS thread per call: concurrent multi-threaded BLAS calls from
    # several threads have returned wrong products with this numpy's OpenBLAS
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(one, range(wl.B * wl.H)))
    return {"heads": wl.B * wl.H, "near_threshold_blocks": sum(r[0] for r in res),
            "flipped_in_band": sum(r[1] for r in res), "differ_outside_band": sum(r[2] for r in res),
            "oracle_routing_s": time.perf_counter() - t0}


def approx_vs(o_s, l_s, od, lsed):
    """Sparse output against dense attention on the same inputs."""
    d = o_s.float() - od.float()
    return {"o_rel_l2": float(d.norm() / od.float().norm()), "o_max_abs": float(d.abs().max()),
            "lse_mean_abs": float((l_s - lsed).abs().mean())}


def peak_for(dtype: str) -> float:
    if dtype == "fp8":
        return 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)   # QK^T fp8, PV bf16
    return PEAK_BF16_TFLOPS


def pool_algorithmic_bytes(wl) -> int:
    """The pool pass's algorithmic bytes: Q, K, V read once (+ the fp8 block
    scales) and the three float32 block-mean tensors written."""
    bh = wl.B * wl.H
    e_qk = {"f32": 4, "bf16": 2, "fp8": 1}[wl.dtype]
    e_v = 4 if wl.dtype == "f32" else 2
    b = bh * wl.N * wl.D * (2 * e_qk + e_v) + 3 * bh * wl.Nb * wl.D * 4
    return b + (2 * bh * wl.Nb * 4 if wl.dtype == "fp8" else 0)


def pool_layout_bytes(wl) -> int:
    """Bytes the pool kernel of this library moves: the algorithmic bytes plus,
    for bf16 V, the bf16 copies of the key/value means (padded to a multiple of
    64 blocks) and V regrouped per 64-key block for the attention kernel."""
    bh, nbp = wl.B * wl.H, (wl.Nb + 63) // 64 * 64
    b = pool_algorithmic_bytes(wl)
    if wl.dtype != "f32":
        b += 2 * bh * nbp * wl.D * 2 + bh * wl.Nb * wl.D * 64 * 2
    return b


def gemm_reference(dev, n: int = 16384, reps: int = 3) -> dict:
    """A plain bf16 GEMM (n x n x n) through torch.matmul, i.e. the vendor's
    tuned GEMM library: the matrix-core rate this GPU sustains for dense bf16
    work in the same run.  Context for the roofline, whose peak is the
    published one (2.5 PFLOP/s at the 2.4 GHz peak clock)."""
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    torch.cuda.empty_cache()
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"what": f"torch.matmul bf16 {n}x{n}x{n}", "ms": ms, "tflops": tflops,
            "frac_of_published_peak": tflops / PEAK_BF16_TFLOPS}


def time_config(name, tau, steps, dense_steps, cpu, inp=None, dev=None, first_order=False):
    """One workload at one tau: sa_pool + sa_forward_pooled timed over `steps`
    calls after a warm-up call, the dense call, density and (cpu) the oracle's
    near-threshold / flipped counts over every head; with first_order (bf16
    only) also the call with the first-order correction (correction = 2),
    whose values the attention call computes per slab of heads."""
    wl = synth.workload(name)
    t0 = time.time()
    if inp is None:
        inp = synth.generate(wl)
    log(f"config {name} tau {tau:g}: inputs in {time.time() - t0:.1f}s")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    qs = inp.q_scale.to(dev) if inp.q_scale is not None else None
    ks = inp.k_scale.to(dev) if inp.k_scale is not None else None
    grid = (wl.T, wl.Hg, wl.Wg)
    correction = wl.correction
    ws = torch.empty(api.sa_workspace_bytes(q, k, v, grid), dtype=torch.uint8, device=dev)
    o = torch.empty(q.shape, dtype=v.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    kept = torch.empty((wl.B, wl.H, wl.Nb), dtype=torch.int32, device=dev)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    mask_np = mask.cpu().numpy().reshape(wl.B * wl.H, wl.Nb, wl.Nb)
    del mask
    f_exact = computed_block_flops(mask_np, wl.N, wl.D)
    f_dense = 4.0 * wl.B * wl.H * wl.N * wl.N * wl.D

    def step():
        api.sa_pool(q, k, v, grid, tau=tau, correction=correction, workspace=ws, q_scale=qs, k_scale=ks)
        api.sa_forward_pooled(q, k, v, grid, tau=tau, correction=correction, workspace=ws, q_scale=qs,
                              k_scale=ks, out=o, lse=lse, kept=kept, want_kept=True)
    step()
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu()), f"fused routing disagrees with sa_route ({name})"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    peak = peak_for(wl.dtype)
    rec = {"workload": name, "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D, "dtype": wl.dtype, "tau": tau,
           "correction": correction, "steps": steps, "ms": ms,
           "computed_block_tflops": f_exact / (ms * 1e-3) / 1e12,
           "frac_peak": f_exact / (ms * 1e-3) / 1e12 / peak, "peak_tflops": peak,
           "dense_equivalent_tflops": f_dense / (ms * 1e-3) / 1e12,
           "block_density": float(mask_np.mean()), "union_inflation": union_inflation(mask_np),
           "computed_block_tflop": f_exact / 1e12}
    if dense_steps > 0:
        od, lsed = torch.empty_like(o), torch.empty_like(lse)
        wsd = torch.empty(max(api.sa_dense_workspace_bytes(q, k, v, grid), 1), dtype=torch.uint8, device=dev)
        api.sa_dense_forward(q, k, v, grid, workspace=wsd, q_scale=qs, k_scale=ks, out=od, lse=lsed)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(dense_steps):
            api.sa_dense_forward(q, k, v, grid, workspace=wsd, q_scale=qs, k_scale=ks, out=od, lse=lsed)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / dense_steps
        rec["dense_ms"] = dms
        rec["dense_tflops"] = f_dense / (dms * 1e-3) / 1e12
        rec["speedup_vs_dense"] = dms / ms
        del od, lsed, wsd
    if first_order and wl.dtype == "bf16":
        del ws
        torch.cuda.empty_cache()
        wsf = torch.empty(api.sa_workspace_bytes(q, k, v, grid, correction=2), dtype=torch.uint8, device=dev)

        def fstep():
            api.sa_pool(q, k, v, grid, tau=tau, correction=2, workspace=wsf)
            api.sa_forward_pooled(q, k, v, grid, tau=tau, correction=2, workspace=wsf, out=o, lse=lse,
                                  kept=kept, want_kept=True)
        fstep()
        torch.cuda.synchronize()
        assert torch.equal(kept.cpu(), kept_r.cpu()), f"fused routing disagrees with sa_route ({name}, first order)"
        e0.record()
        for _ in range(steps):
            fstep()
        e1.record()
        torch.cuda.synchronize()
        fms = e0.elapsed_time(e1) / steps
        per = api.first_order_slab(q, v)
        rec["first_order"] = {"ms": fms, "time_vs_mean_copies": fms / ms, "heads_per_slab": per,
                              "slabs": -(-(wl.B * wl.H) // per), "workspace_gib": wsf.numel() / 2 ** 30}
        del wsf
        ws = None
        log(f"config {name} tau {tau:g}: first order {fms:.2f} ms ({fms / ms:.3f}x)")
    del q, k, v, ws, o, lse, kept
    torch.cuda.empty_cache()
    if cpu:
        rec["routing_vs_oracle"] = route_band_counts(inp, wl, tau, mask_np)
    log(f"config {name} tau {tau:g}: {ms:.2f} ms, density {rec['block_density']:.3f}")
    return rec


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="720p", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--no-correction", action="store_true")
    ap.add_argument("--dense-steps", type=int, default=2)
    ap.add_argument("--cpu-heads", type=int, default=1, help="whole heads of oracle work in cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--budgets", default="0.9,0.8",
                    help="fixed-budget routing sparsities to time as well (comma list, '' for none)")
    ap.add_argument("--budget-steps", type=int, default=5)
    ap.add_argument("--tiles", default="4x4x4,1x8x8",
                    help="3-D tile orders (t x h x w, product 64) to time at the same tau ('' for none)")
    ap.add_argument("--no-first-order", dest="first_order", action="store_false",
                    help="skip timing the first-order correction (correction = 2)")
    ap.add_argument("--configs", default="720p:4,720p:8,480p:4,1080p:4,720p_cfg_fp8:4",
                    help="other workloads to time as name:tau (comma list, '' for none)")
    ap.add_argument("--config-steps", type=int, default=3)
    ap.add_argument("--first-order-configs", default="1080p",
                    help="workloads of --configs whose call with the first-order correction is timed too")
    ap.add_argument("--no-gemm-reference", dest="gemm_reference", action="store_false",
                    help="skip the bf16 library GEMM timed as the matrix-core reference")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device-to-device copy (reference for the PMC byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the path shards by (batch, head) with no exchange, "
              "and runs on more than one GPU are not supported. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    wl = synth.workload(args.workload)
    tau = args.tau if args.tau is not None else wl.taus[0]
    correction = wl.correction and not args.no_correction
    grid = (wl.T, wl.Hg, wl.Wg)
    t0 = time.time()
    inp = synth.generate(wl)
    log(f"generated {wl.name} B{wl.B} H{wl.H} N{wl.N} D{wl.D} {wl.dtype} in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    qs = inp.q_scale.to(dev) if inp.q_scale is not None else None
    ks = inp.k_scale.to(dev) if inp.k_scale is not None else None
    ws = torch.empty(api.sa_workspace_bytes(q, k, v, grid), dtype=torch.uint8, device=dev)
    o = torch.empty(q.shape, dtype=v.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    kept = torch.empty((wl.B, wl.H, wl.Nb), dtype=torch.int32, device=dev)

    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    mask_np = mask.cpu().numpy().reshape(wl.B * wl.H, wl.Nb, wl.Nb)
    del mask
    f_exact = computed_block_flops(mask_np, wl.N, wl.D)
    f_corr = correction_flops(mask_np, wl.N, wl.D) if correction else 0.0
    f_dense = 4.0 * wl.B * wl.H * wl.N * wl.N * wl.D
    density = float(mask_np.mean())

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        api.sa_pool(q, k, v, grid, tau=tau, correction=correction, workspace=ws, q_scale=qs, k_scale=ks)
        if ev is not None:
            ev[1].record()
        api.sa_forward_pooled(q, k, v, grid, tau=tau, correction=correction, workspace=ws, q_scale=qs,
                              k_scale=ks, out=o, lse=lse, kept=kept, want_kept=True)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    pool_ms = [e[0].elapsed_time(e[1]) for e in evs]
    fused_ms = [e[1].elapsed_time(e[2]) for e in evs]
    assert torch.equal(kept.cpu(), kept_r.cpu()), "fused routing disagrees with sa_route"

    value = f_exact / (ms_step * 1e-3) / 1e12
    fused_avg = float(np.mean(fused_ms))
    achieved = f_exact / (fused_avg * 1e-3) / 1e12
    peak = peak_for(wl.dtype)
    pool_bytes = pool_algorithmic_bytes(wl)
    pool_lbytes = pool_layout_bytes(wl)
    pool_avg = float(np.mean(pool_ms))

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_src_sha256") == kernel_source_hash() and tr.get("workload") == wl.name \
                and float(tr.get("tau", -1)) == tau:
            traffic = tr.get("bytes_per_launch")

    # dense path at the same shape (the tau = inf baseline)
    dense = None
    od = lsed = None
    if args.dense_steps > 0:
        wsd = torch.empty(max(api.sa_dense_workspace_bytes(q, k, v, grid), 1), dtype=torch.uint8, device=dev)
        od = torch.empty_like(o)
        lsed = torch.empty_like(lse)
        api.sa_dense_forward(q, k, v, grid, workspace=wsd, q_scale=qs, k_scale=ks, out=od, lse=lsed)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.dense_steps):
            api.sa_dense_forward(q, k, v, grid, workspace=wsd, q_scale=qs, k_scale=ks, out=od, lse=lsed)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / args.dense_steps
        dense = {"ms": dms, "tflops": f_dense / (dms * 1e-3) / 1e12,
                 "frac_peak": f_dense / (dms * 1e-3) / 1e12 / peak, "sparse_speedup": dms / ms_step}

        # what the method approximates: the sparse output against dense
        # attention on the same inputs, with the correction as configured and
        # toggled (the error the correction of the skipped blocks removes)
        o_t, l_t = api.sa_forward(q, k, v, grid, tau=tau, correction=not correction, workspace=ws,
                                  q_scale=qs, k_scale=ks)[:2]
        torch.cuda.synchronize()
        dense["approx_vs_dense"] = {"tau": tau, ("correction_on" if correction else "correction_off"):
                                    approx_vs(o, lse, od, lsed),
                                    ("correction_off" if correction else "correction_on"):
                                    approx_vs(o_t, l_t, od, lsed)}
        del wsd, o_t, l_t

    # first-order correction of the skipped blocks (correction = 2) at the
    # same tau: the attention call computes one first-order value per (query
    # block, key block) for a slab of heads at a time, then runs the fused
    # kernel on that slab, whose correction tiles read them
    first_order = None
    if wl.dtype == "bf16" and args.first_order:
        wsf = torch.empty(api.sa_workspace_bytes(q, k, v, grid, correction=2), dtype=torch.uint8, device=dev)
        of, lsef = torch.empty_like(o), torch.empty_like(lse)

        def fstep(ev=None):
            if ev is not None:
                ev[0].record()
            api.sa_pool(q, k, v, grid, tau=tau, correction=2, workspace=wsf)
            if ev is not None:
                ev[1].record()
            api.sa_forward_pooled(q, k, v, grid, tau=tau, correction=2, workspace=wsf, out=of, lse=lsef,
                                  kept=kept, want_kept=True)
            if ev is not None:
                ev[2].record()
        fstep()
        torch.cuda.synchronize()
        assert torch.equal(kept.cpu(), kept_r.cpu()), "fused routing disagrees with sa_route (first order)"
        fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.budget_steps)]
        for i in range(args.budget_steps):
            fstep(fevs[i])
        torch.cuda.synchronize()
        fpool = float(np.mean([e[0].elapsed_time(e[1]) for e in fevs]))
        fattn = float(np.mean([e[1].elapsed_time(e[2]) for e in fevs]))
        first_order = {"tau": tau, "ms": fpool + fattn, "pool_ms": fpool,
                       "values_and_fused_kernel_ms": fattn,
                       "values_by_difference_ms": fattn - fused_avg,
                       "workspace_gib": wsf.numel() / 2 ** 30,
                       "heads_per_slab": api.first_order_slab(q, v),
                       "time_vs_mean_copies": (fpool + fattn) / ms_step,
                       "approx_vs_dense": approx_vs(of, lsef, od, lsed) if od is not None else None}
        del wsf
        if od is not None:
            # with blocks over 4x4x4 tiles of the grid the keys of a block lie
            # closer together, and the first-order term matters more
            tiled_err = {"tile": [4, 4, 4], "tau": tau}
            for name, corr in (("mean_copies", 1), ("first_order", 2)):
                api.sa_forward(q, k, v, grid, tau=tau, correction=corr, tile=(4, 4, 4), out=of, lse=lsef)
                torch.cuda.synchronize()
                tiled_err[name] = approx_vs(of, lsef, od, lsed)
            first_order["approx_vs_dense_tiled"] = tiled_err
        log(f"first-order correction: pool {fpool:.2f} ms, values + fused {fattn:.2f} ms")
        del of, lsef
    del od, lsed

    # fixed-budget routing (topk blocks per query block) at the same shape
    budgets = []
    ob, lseb = torch.empty_like(o), torch.empty_like(lse)   # keeps o / lse of the tau run intact
    for sp in [float(x) for x in args.budgets.split(",") if x.strip()]:
        topk = api.budget_blocks(sp, wl.N)
        bmask, bkept = api.sa_route(q, k, v, grid, topk=topk, q_scale=qs, k_scale=ks)
        torch.cuda.synchronize()
        bmask_np = bmask.cpu().numpy().reshape(wl.B * wl.H, wl.Nb, wl.Nb)
        del bmask
        bf = computed_block_flops(bmask_np, wl.N, wl.D)

        def bstep():
            api.sa_pool(q, k, v, grid, topk=topk, correction=correction, workspace=ws, q_scale=qs, k_scale=ks)
            api.sa_forward_pooled(q, k, v, grid, topk=topk, correction=correction, workspace=ws, q_scale=qs,
                                  k_scale=ks, out=ob, lse=lseb, kept=kept, want_kept=True)
        bstep()
        torch.cuda.synchronize()
        assert torch.equal(kept.cpu(), bkept.cpu()), "fused routing disagrees with sa_route (topk)"
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.budget_steps):
            bstep()
        e1.record()
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / args.budget_steps
        budgets.append({"sparsity": sp, "topk": topk, "ms": bms,
                        "computed_block_tflops": bf / (bms * 1e-3) / 1e12,
                        "frac_mfma_peak": bf / (bms * 1e-3) / 1e12 / peak,
                        "block_density": float(bmask_np.mean()),
                        "union_inflation": union_inflation(bmask_np),
                        "speedup_vs_dense": (dense["ms"] / bms) if dense else None})
        log(f"budget sparsity {sp}: topk {topk}, {bms:.2f} ms")

    # fused Q/K producer step (norm + rotary + pool) in place of the pool: the
    # workload's Q/K stand in for the raw projections
    producer = None
    if wl.dtype == "bf16":
        gq = torch.ones(wl.D, dtype=torch.float32, device=dev)
        qo, ko = torch.empty_like(q), torch.empty_like(k)
        wsp = torch.empty_like(ws)
        api.sa_qk_prologue(q, k, v, grid, gq, gq, tau=tau, workspace=wsp, q_out=qo, k_out=ko)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.budget_steps):
            api.sa_qk_prologue(q, k, v, grid, gq, gq, tau=tau, workspace=wsp, q_out=qo, k_out=ko)
        e1.record()
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / args.budget_steps
        pbytes = pool_lbytes + 2 * wl.B * wl.H * wl.N * wl.D * 2      # + Q and K written back
        producer = {"ms": pms, "gbs": pbytes / (pms * 1e-3) / 1e9,
                    "frac_hbm": pbytes / (pms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": pbytes,
                    "unfused_extra_bytes": 2 * wl.B * wl.H * wl.N * wl.D * 2}
        log(f"fused producer: {pms:.3f} ms")
        del qo, ko, wsp

    # 3-D tile token order (blocks are tiles of the token grid) at the same tau
    tiled = []
    for spec in [x for x in args.tiles.split(",") if x.strip()]:
        tile = tuple(int(t) for t in spec.lower().split("x"))
        if wl.dtype == "fp8":
            break                       # fp8 block scales belong to raster blocks
        wst = torch.empty(api.sa_workspace_bytes(q, k, v, grid, tile=tile), dtype=torch.uint8, device=dev)
        tmask, tkept = api.sa_route(q, k, v, grid, tau=tau, tile=tile, workspace=wst)
        torch.cuda.synchronize()
        tmask_np = tmask.cpu().numpy().reshape(wl.B * wl.H, wl.Nb, wl.Nb)
        del tmask
        tf = computed_block_flops(tmask_np, wl.N, wl.D)

        def tstep(ev=None):
            if ev is not None:
                ev[0].record()
            api.sa_pool(q, k, v, grid, tau=tau, correction=correction, workspace=wst, tile=tile)
            if ev is not None:
                ev[1].record()
            api.sa_forward_pooled(q, k, v, grid, tau=tau, correction=correction, workspace=wst, tile=tile,
                                  out=ob, lse=lseb, kept=kept, want_kept=True)
            if ev is not None:
                ev[2].record()
        tstep()
        torch.cuda.synchronize()
        assert torch.equal(kept.cpu(), tkept.cpu()), "fused routing disagrees with sa_route (tiles)"
        tevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.budget_steps)]
        for i in range(args.budget_steps):
            tstep(tevs[i])
        torch.cuda.synchronize()
        tpool = float(np.mean([e[0].elapsed_time(e[1]) for e in tevs]))
        tms = float(np.mean([e[0].elapsed_time(e[2]) for e in tevs]))
        tiled.append({"tile": list(tile), "tau": tau, "ms": tms, "pool_ms": tpool,
                      "computed_block_tflops": tf / (tms * 1e-3) / 1e12,
                      "block_density": float(tmask_np.mean()),
                      "union_inflation": union_inflation(tmask_np),
                      "speedup_vs_dense": (dense["ms"] / tms) if dense else None})
        log(f"tile {spec}: density {tmask_np.mean():.3f}, {tms:.2f} ms")
        del wst

    # a 1 GiB device-to-device copy: the streaming rate the HBM-bound pool is
    # measured against (and, with --calibrate-copy, the PMC byte reference)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    copy_ms = None
    if not args.calibrate_copy:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_ms = e0.elapsed_time(e1) / 5
    del src, dst

    gemm_ref = gemm_reference(dev) if args.gemm_reference else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, wl, tau, o, args.cpu_heads)
        cpu["routing_vs_oracle"] = route_band_counts(inp, wl, tau, mask_np)
    del q, k, v, ws, o, lse, kept, ob, lseb
    torch.cuda.empty_cache()

    configs = []
    for spec in [x for x in args.configs.split(",") if x.strip()]:
        cname, ctau = spec.split(":")
        same = cname == wl.name
        fo_names = [x.strip() for x in args.first_order_configs.split(",") if x.strip()]
        configs.append(time_config(cname, float(ctau), args.config_steps, 1, not args.no_cpu_baseline,
                                   inp=inp if same else None, dev=dev, first_order=cname in fo_names))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "fp8": "fp8e4m3-qk/bf16-pv"}[wl.dtype],
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name} video-DiT self-attention: B{wl.B} H{wl.H} grid {wl.T}x{wl.Hg}x{wl.Wg} "
                         f"N{wl.N} D{wl.D} {wl.dtype}, block 64, tau {tau:g}, correction "
                         f"{'on' if correction else 'off'}"),
            "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D, "tau": tau, "correction": correction,
            "parallelism": "single GPU (heads independent)",
        },
        "frac_mfma_peak": value / peak,
        "block_density": density,
        "union_inflation": union_inflation(mask_np),
        "work_density": f_exact / f_dense,
        "computed_block_tflop": f_exact / 1e12,
        "correction_tflop": f_corr / 1e12,
        "dense_equivalent_tflops": f_dense / (ms_step * 1e-3) / 1e12,
        "pool": {"ms": pool_avg, "gbs": pool_bytes / (pool_avg * 1e-3) / 1e9,
                 "frac_hbm": pool_bytes / (pool_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": pool_bytes,
                 "bytes_kind": "algorithmic: Q, K, V read once + float32 block means written",
                 "layout_bytes": pool_lbytes, "layout_gbs": pool_lbytes / (pool_avg * 1e-3) / 1e9,
                 "copy_1gib_gbs": (2 * (1 << 30) / (copy_ms * 1e-3) / 1e9) if copy_ms else None},
        "fused_kernel_ms": fused_avg,
        "ms_per_call_median": float(np.median(np.add(pool_ms, fused_ms))),
        "ms_per_call_min": float(np.min(np.add(pool_ms, fused_ms))),
        "ms_per_call_p90": float(np.percentile(np.add(pool_ms, fused_ms), 90)),
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": "attn_kernel (fused route + correction + sparse flash attention)",
                     "achieved_incl_correction": (f_exact + f_corr) / (fused_avg * 1e-3) / 1e12},
        "dense": dense,
        "fixed_budget": budgets,
        "tile_order": tiled,
        "fused_producer": producer,
        "first_order": first_order,
        "configs": configs,
        "gemm_reference": gemm_ref,
        "cpu_baseline": cpu,
        "kernel_src": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
