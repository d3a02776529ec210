"""GPU parity of the first-order correction (correction = 2) against the CPU
oracle.

* seeded cases spanning several tiles and a ragged tail: D = 128 and 64,
  threshold and fixed budget, raster and 3-D tile order, batch and heads
  above one, explicit scale, bf16, float32 and fp8 Q/K inputs: masks and
  every row's O and LSE against the oracle's first-order model (float32 at
  its 1e-5 bounds, fp8 at its 4e-2 bound);
* the first-order values themselves (the workspace section the attention
  call fills, one slab of heads at a time; at these sizes one slab holds
  every head) against oracle.first_order_value for every (query block, key
  block) pair of a case, padding rows zero;
* LSE against the mean copies' run on the same inputs: the first-order model
  changes the skipped blocks' values only, and the kernel takes the same
  weights, so the two agree bit for bit; with tau = inf (nothing skipped) O
  agrees bit for bit too;
* the fused producer step followed by the first-order path;
* the maximum sequence length (N = 262,144, Nb = 4096);
* the 720p size (B = 1, H = 40, 21 x 45 x 80, bf16) at tau = 2, the
  configuration the benchmark times for this mode (2 slabs of 20 heads):
  masks of every head, O and LSE of sampled query blocks of four heads; the
  720p CFG fp8 configuration (B = 2) at tau = 4, two heads; and the 1080p
  configuration (B = 1, H = 32, 21 x 68 x 120, tau = 4; 8 slabs of 4 heads),
  four heads from different slabs.
"""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from oracle import attention as orc
from tests.parity import mask_check, mask_check_topk, oracle_map, output_check, say, to_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, (T, Hg, Wg), D, tau, topk, tile, scale, seed
    ("d128_tau1", 1, 2, (3, 10, 13), 128, 1.0, 0, None, 0.0, 31),
    ("d128_tau0", 2, 1, (2, 16, 20), 128, 0.0, 0, None, 0.0, 32),
    ("d128_topk3", 1, 3, (4, 9, 15), 128, 0.0, 3, None, 0.0, 33),
    ("d64_tau2", 2, 2, (3, 12, 12), 64, 2.0, 0, None, 0.0, 34),
    ("d64_topk2_scale", 1, 2, (2, 14, 11), 64, 0.0, 2, None, 0.09, 35),
    ("tiles_2x4x8", 1, 2, (4, 8, 17), 128, 0.5, 0, (2, 4, 8), 0.0, 36),
    ("tiles_4x4x4_topk", 1, 1, (5, 9, 9), 128, 0.0, 4, (4, 4, 4), 0.0, 37),
    ("one_block", 1, 1, (1, 5, 9), 128, 0.0, 0, None, 0.0, 38),
    # float32 inputs: the float32 path, at its tighter tolerances
    ("f32_d64_tau1", 1, 2, (2, 12, 13), 64, 1.0, 0, None, 0.0, 39, "f32"),
    ("f32_d128_topk3_tiles", 2, 1, (4, 8, 12), 128, 0.0, 3, (2, 4, 8), 0.0, 40, "f32"),
    # fp8 e4m3 Q/K with block scales, bf16 V
    ("fp8_d128_tau1", 2, 1, (3, 10, 13), 128, 1.0, 0, None, 0.0, 41, "fp8"),
    ("fp8_d64_topk2", 1, 2, (2, 14, 11), 64, 0.0, 2, None, 0.0, 42, "fp8"),
]


def _run(case, corr):
    name, B, H, grid, D, tau, topk, tile, scale, seed = case[:10]
    dtype = case[10] if len(case) > 10 else "bf16"
    wl = synth.Workload(name, B, H, *grid, D, dtype, (tau,), True, seed=seed)
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    kw = dict(tau=tau, topk=topk, tile=tile, scale=scale, q_scale=qs, k_scale=ks)
    ws = api.sa_pool(q, k, v, grid, correction=corr, **kw)
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, workspace=ws, correction=corr, want_kept=True, **kw)
    return wl, inp, (q, k, v, qs, ks), ws, o, lse, kept


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_first_order_parity(case):
    name, B, H, grid, D, tau, topk, tile, scale, seed = case[:10]
    say(f"case {case}")
    wl, inp, (q, k, v, qs, ks), ws, o, lse, kept = _run(case, 2)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau, topk=topk, tile=tile, scale=scale, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    m = mask.cpu().numpy()
    order = None if tile is None else orc.tile_order(*grid, tile)
    sc = scale if scale > 0 else None
    for b in range(B):
        for h in range(H):
            if topk:
                keep, _, _ = mask_check_topk(inp, b, h, m[b, h], topk, scale=sc, order=order)
            else:
                keep, _, _ = mask_check(inp, b, h, m[b, h], tau, scale=sc, order=order)
            st = output_check(inp, b, h, o, lse, keep, tau, 2, scale=sc, order=order)
            say(f"  head ({b},{h}): {st}")


VALUE_CASES = [CASES[0], CASES[3], CASES[5]] + [c for c in CASES if len(c) > 10 and c[10] == "fp8"]


@pytest.mark.parametrize("case", VALUE_CASES, ids=[c[0] for c in VALUE_CASES])
def test_first_order_values(case):
    """The workspace's first-order values against the oracle, every pair
    (fp8: of the dequantised keys)."""
    name, B, H, grid, D, tau, topk, tile, scale, seed = case[:10]
    say(f"case {case}")
    wl, inp, (q, k, v, qs, ks), ws, _, _, _ = _run(case, 2)
    torch.cuda.synchronize()
    off = api.sa_workspace_bytes(q, k, v, grid, qs, ks, tile=tile, correction=1)
    Nb = wl.Nb
    Nbp = (Nb + 63) // 64 * 64
    n = B * H * Nb * Nbp * D
    assert ws.numel() - off >= 2 * n
    vp = ws[off:off + 2 * n].view(torch.bfloat16).view(B, H, Nb, Nbp, D).float().cpu().numpy()
    assert (vp[:, :, :, Nb:, :] == 0).all(), "padding rows are not zero"
    s = scale if scale > 0 else 1.0 / math.sqrt(D)
    order = None if tile is None else np.asarray(orc.tile_order(*grid, tile))
    ranges = orc.block_ranges(wl.N, 64)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = inp.head64(b, h)
            if order is not None:
                qh, kh, vh = qh[order], kh[order], vh[order]
            ref = np.empty((Nb, Nb, D))
            mag = np.empty((Nb, Nb, D))
            for I in range(Nb):
                qbar = qh[slice(*ranges[I])].mean(axis=0)
                for J in range(Nb):
                    kJ, vJ = kh[slice(*ranges[J])], vh[slice(*ranges[J])]
                    ref[I, J] = orc.first_order_value(qbar, kJ, vJ, s)
                    # (s / n_J) sum_j |v_j| sum_d |qbar_d| |d_jd|: the scale of the
                    # rounding inside the first-order term
                    mag[I, J] = s * (np.abs(kJ - kJ.mean(axis=0)) @ np.abs(qbar)) @ np.abs(vJ) / kJ.shape[0]
            got = vp[b, h, :, :Nb, :]
            err = np.abs(got - ref)
            # the stored value is bf16 (2^-9 relative); inside the first-order term
            # qbar and each centred score are rounded to bf16 (2^-9 each, relative
            # to the terms of the sum, hence the absolute-value sum mag); 2x margin
            bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -7 * mag + 1e-6
            say(f"  head ({b},{h}): max err {err.max():.3e}, max |term| sum {mag.max():.3e}, "
                f"worst err/bound {(err / bound).max():.3f}")
            assert (err <= bound).all()


F32_CASES = [c for c in CASES if len(c) > 10 and c[10] == "f32"]


@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_first_order_values_f32(case):
    """Float32 path: its values section ([BH][Nb][Nb][D] float) against the
    oracle, every pair, at float32 rounding."""
    name, B, H, grid, D, tau, topk, tile, scale, seed = case[:10]
    say(f"case {case}")
    wl, inp, (q, k, v, qs, ks), ws, _, _, _ = _run(case, 2)
    torch.cuda.synchronize()
    off = api.sa_workspace_bytes(q, k, v, grid, tile=tile, correction=1)
    Nb = wl.Nb
    n = B * H * Nb * Nb * D
    vp = ws[off:off + 4 * n].view(torch.float32).view(B, H, Nb, Nb, D).cpu().numpy().astype(np.float64)
    s = scale if scale > 0 else 1.0 / math.sqrt(D)
    order = None if tile is None else np.asarray(orc.tile_order(*grid, tile))
    ranges = orc.block_ranges(wl.N, 64)
    for b in range(B):
        for h in range(H):
            qh, kh, vh = inp.head64(b, h)
            if order is not None:
                qh, kh, vh = qh[order], kh[order], vh[order]
            worst = 0.0
            for I in range(Nb):
                qbar = qh[slice(*ranges[I])].mean(axis=0)
                for J in range(Nb):
                    kJ, vJ = kh[slice(*ranges[J])], vh[slice(*ranges[J])]
                    ref = orc.first_order_value(qbar, kJ, vJ, s)
                    mag = s * (np.abs(kJ - kJ.mean(axis=0)) @ np.abs(qbar)) @ np.abs(vJ) / kJ.shape[0]
                    bound = 1e-6 * (np.abs(ref) + mag) + 1e-7
                    err = np.abs(vp[b, h, I, J] - ref)
                    worst = max(worst, float((err / bound).max()))
                    assert (err <= bound).all(), (b, h, I, J, float(err.max()))
            say(f"  head ({b},{h}): worst err/bound {worst:.3f}")


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[4]], ids=[CASES[i][0] for i in (0, 2, 4)])
def test_lse_equals_mean_copies(case):
    say(f"case {case}")
    _, _, _, _, o2, lse2, _ = _run(case, 2)
    _, _, _, _, o1, lse1, _ = _run(case, 1)
    torch.cuda.synchronize()
    assert torch.equal(lse1, lse2)
    assert not torch.equal(o1, o2)


def test_keep_all_equals_mean_copies():
    """tau = inf skips nothing: the first-order run equals the mean copies' bit
    for bit (its correction tiles are all masked)."""
    case = ("keep_all", 1, 2, (3, 10, 13), 128, math.inf, 0, None, 0.0, 44)
    say(f"case {case}")
    _, _, _, _, o2, lse2, kept = _run(case, 2)
    _, _, _, _, o1, lse1, _ = _run(case, 1)
    torch.cuda.synchronize()
    assert (kept.cpu() == kept.shape[-1]).all()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)


def test_producer_then_first_order():
    """sa_qk_prologue leaves the workspace sa_pool would write from its
    outputs (everything in front of the first-order values, which the
    attention call computes), and the first-order attention on the two
    workspaces agrees bit for bit (the producer's own parity is covered with
    the producer's tests)."""
    B, H, grid, D = 1, 3, (3, 8, 12), 128
    N = grid[0] * grid[1] * grid[2]
    say(f"case producer B={B} H={H} grid={grid}")
    g = torch.Generator().manual_seed(41)
    xq = (torch.randn((B, H, N, D), generator=g) * 2).to(torch.bfloat16)
    xk = (torch.randn((B, H, N, D), generator=g) * 2).to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=g).to(torch.bfloat16)
    qg = (1 + 0.1 * torch.randn(D, generator=g)).float()
    kg = (1 + 0.1 * torch.randn(D, generator=g)).float()
    dev = torch.device("cuda:0")
    xq, xk, v, qg, kg = (t.to(dev) for t in (xq, xk, v, qg, kg))
    qo, ko, ws = api.sa_qk_prologue(xq, xk, v, grid, qg, kg, tau=1.0, correction=2)
    ws2 = api.sa_pool(qo, ko, v, grid, tau=1.0, correction=2)
    torch.cuda.synchronize()
    off = api.sa_workspace_bytes(qo, ko, v, grid, correction=1)
    assert torch.equal(ws[:off], ws2[:off])
    o1, l1, _ = api.sa_forward_pooled(qo, ko, v, grid, tau=1.0, correction=2, workspace=ws)
    o2, l2, _ = api.sa_forward_pooled(qo, ko, v, grid, tau=1.0, correction=2, workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_first_order_maximum_sequence_length():
    """N = 262,144 tokens (Nb = 4096, the on-chip routing limit; 64 correction
    tiles per query block), sampled query blocks incl. the last ones."""
    grid = (64, 64, 64)
    wl = synth.Workload("max_first_order", 1, 1, *grid, 128, "bf16", (2.0,), True, seed=43)
    assert wl.N == api.MAX_N
    say("case first-order N = MAX_N")
    inp = synth.generate(wl)
    q, k, v, _, _ = to_gpu(inp)
    ws = api.sa_pool(q, k, v, grid, tau=2.0, correction=2)
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, tau=2.0, correction=2, workspace=ws, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=2.0)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    del ws
    keep, _, _ = mask_check(inp, 0, 0, mask[0, 0].cpu().numpy(), 2.0)
    st = output_check(inp, 0, 0, o, lse, keep, 2.0, 2, qblocks=[0, 2047, 4094, 4095])
    say(f"  {st}")


_WL = None


def _inputs_720p():
    global _WL
    if _WL is None:
        wl = synth.workload("720p")
        _WL = (wl, synth.generate(wl))
    return _WL


def test_first_order_720p_cfg_fp8():
    """The 720p CFG configuration (B = 2, H = 40, fp8 e4m3 Q/K with block
    scales, bf16 V) at its tau = 4 with the first-order correction: kept
    counts of every head against sa_route, masks and sampled query blocks of
    two heads (one per CFG batch) against the oracle."""
    wl = synth.workload("720p_cfg_fp8")
    tau = wl.taus[0]
    say(f"case 720p CFG fp8 first-order tau={tau}")
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    kw = dict(tau=tau, q_scale=qs, k_scale=ks)
    ws = api.sa_pool(q, k, v, grid, correction=2, **kw)
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, correction=2, workspace=ws, want_kept=True, **kw)
    mask, kept_r = api.sa_route(q, k, v, grid, **kw)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    del ws, q, k, v
    for (b, h) in [(0, 0), (1, wl.H - 1)]:
        keep, _, _ = mask_check(inp, b, h, mask[b, h].cpu().numpy(), tau)
        st = output_check(inp, b, h, o, lse, keep, tau, 2, qblocks=[0, 600, wl.Nb - 1])
        say(f"  head ({b},{h}): {st}")


def test_first_order_720p():
    wl, inp = _inputs_720p()
    tau = 2.0
    say(f"case 720p first-order tau={tau}")
    q, k, v, _, _ = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    ws = api.sa_pool(q, k, v, grid, tau=tau, correction=2)
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, tau=tau, correction=2, workspace=ws, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    del ws, q, k, v
    mask_np = mask.cpu().numpy()
    del mask
    heads = [(0, h) for h in range(wl.H)]
    res = oracle_map(lambda bh: mask_check(inp, bh[0], bh[1], mask_np[bh], tau), heads)
    say(f"  masks ok for {len(heads)} heads; density {mask_np.mean():.3f}")
    rng = np.random.default_rng(11)
    sample = sorted({(0, 0), (0, wl.H - 1), (0, int(rng.integers(wl.H))), (0, int(rng.integers(wl.H)))})
    for (b, h) in sample:
        keep = res[heads.index((b, h))][0]
        qb = {0, wl.Nb - 1, int(rng.integers(wl.Nb)), int(rng.integers(wl.Nb))}
        st = output_check(inp, b, h, o, lse, keep, tau, 2, qblocks=qb)
        say(f"  head ({b},{h}) blocks {sorted(qb)}: {st}")


def test_first_order_1080p():
    """The 1080p configuration with the first-order correction: its values
    take 1.84 GB per head, so the call runs 8 slabs of 4 heads.  Kept
    counts of every head against sa_route; masks and sampled query blocks of
    heads from the first, a middle and the last slab against the oracle."""
    wl = synth.workload("1080p")
    tau = wl.taus[0]
    say(f"case 1080p first-order tau={tau}")
    inp = synth.generate(wl)
    q, k, v, _, _ = to_gpu(inp)
    assert api.first_order_slab(q, v) == 4
    grid = (wl.T, wl.Hg, wl.Wg)
    ws = api.sa_pool(q, k, v, grid, tau=tau, correction=2)
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, tau=tau, correction=2, workspace=ws, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    del ws, q, k, v
    for (b, h) in [(0, 0), (0, 5), (0, 17), (0, wl.H - 1)]:
        keep, _, _ = mask_check(inp, b, h, mask[b, h].cpu().numpy(), tau)
        st = output_check(inp, b, h, o, lse, keep, tau, 2, qblocks=[0, 1339, wl.Nb - 1])
        say(f"  head ({b},{h}): {st}")
