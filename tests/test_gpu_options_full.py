"""GPU parity at the full 720p size (B = 1, H = 40, 21 x 45 x 80 tokens, D =
128, bf16) for the launch configurations the benchmark times besides the
threshold headline: fixed-budget routing at sparsity 0.9 and 0.8, the 3-D
tile orders 4x4x4 and 1x8x8 at tau = 2, and the fused Q/K producer step.

Masks are compared for every head; O and LSE on sampled outputs the oracle
computes one query block at a time (heads 0, 39 and two seeded random heads;
first, ragged last and two random query blocks each).  The producer's Q/K are
compared with the oracle on sampled tokens (grid corners and seeded random
tokens, so the largest rotation angles are covered), its workspace bit for bit
with sa_pool run on its own outputs.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from oracle import attention as orc
from oracle import prologue as pro
from tests.parity import mask_check, mask_check_topk, oracle_map, output_check, say, to_gpu

pytestmark = pytest.mark.gpu

_WL = None


def _inputs():
    global _WL
    if _WL is None:
        wl = synth.workload("720p")
        _WL = (wl, synth.generate(wl))
    return _WL


def _sample(wl, rng):
    heads = [(0, h) for h in range(wl.H)]
    sample = {(0, 0), (0, wl.H - 1)}
    while len(sample) < 4:
        sample.add(heads[int(rng.integers(len(heads)))])
    return sorted(sample)


def _check_all(inp, mask_np, check, o, lse, tau, order=None, seed=7):
    wl = inp.wl
    heads = [(0, h) for h in range(wl.H)]
    res = oracle_map(lambda bh: check(bh, mask_np[bh]), heads)
    say(f"  masks ok for {len(heads)} heads; density {mask_np.mean():.3f}; "
        f"near-threshold {sum(r[1] for r in res)}, flipped {sum(r[2] for r in res)}")
    rng = np.random.default_rng(seed)
    for (b, h) in _sample(wl, rng):
        keep = res[heads.index((b, h))][0]
        qb = {0, wl.Nb - 1, int(rng.integers(wl.Nb)), int(rng.integers(wl.Nb))}
        st = output_check(inp, b, h, o, lse, keep, tau, wl.correction, qblocks=qb, order=order)
        say(f"  head ({b},{h}) blocks {sorted(qb)}: {st}")


@pytest.mark.parametrize("sparsity", [0.9, 0.8])
def test_fixed_budget_720p(sparsity):
    wl, inp = _inputs()
    topk = api.budget_blocks(sparsity, wl.N)
    say(f"case 720p fixed budget sparsity={sparsity} topk={topk}")
    q, k, v, _, _ = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    ws = api.sa_pool(q, k, v, grid, topk=topk)
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, topk=topk, workspace=ws, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, topk=topk)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    assert (kept_r.cpu().numpy() == topk).all()
    del ws, q, k, v
    mask_np = mask.cpu().numpy()
    del mask
    _check_all(inp, mask_np, lambda bh, m: mask_check_topk(inp, bh[0], bh[1], m, topk), o, lse, 0.0)


@pytest.mark.parametrize("tile", [(4, 4, 4), (1, 8, 8)], ids=["4x4x4", "1x8x8"])
def test_tile_order_720p(tile):
    wl, inp = _inputs()
    tau = 2.0
    say(f"case 720p tile={tile} tau={tau}")
    q, k, v, _, _ = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    ws = api.sa_pool(q, k, v, grid, tau=tau, tile=tile)
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, tau=tau, tile=tile, workspace=ws, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau, tile=tile)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    del ws, q, k, v
    mask_np = mask.cpu().numpy()
    del mask
    order = orc.tile_order(wl.T, wl.Hg, wl.Wg, tile)
    _check_all(inp, mask_np, lambda bh, m: mask_check(inp, bh[0], bh[1], m, tau, order=order), o, lse, tau,
               order=order)


def test_producer_720p():
    wl, inp = _inputs()
    tau = 2.0
    say("case 720p fused producer tau=2")
    rng = np.random.default_rng(17)
    gq = torch.from_numpy(rng.uniform(0.5, 1.5, size=wl.D).astype(np.float32))
    gk = torch.from_numpy(rng.uniform(0.5, 1.5, size=wl.D).astype(np.float32))
    xq, xk, v, _, _ = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    q, k, ws = api.sa_qk_prologue(xq, xk, v, grid, gq.cuda(), gk.cuda(), tau=tau)
    torch.cuda.synchronize()
    del xq, xk
    # 1. Q/K on sampled tokens against the oracle (one bf16 rounding of a float32 result)
    hw = wl.Hg * wl.Wg
    corners = [0, wl.Wg - 1, hw - 1, (wl.T - 1) * hw, wl.N - wl.Wg, wl.N - 1]
    toks = np.array(sorted(set(corners + rng.integers(0, wl.N, 58).tolist())))
    ang = pro.rope_angles(wl.T, wl.Hg, wl.Wg, wl.D, 10000.0)[toks]
    worst = 0.0
    for h in (0, 13, wl.H - 1):
        for x_raw, g, y_gpu in ((inp.q, gq, q), (inp.k, gk, k)):
            x = x_raw[0, h, toks].to(torch.float64).numpy()
            y_ref = pro.apply_rope(pro.rms_norm(x, g.numpy().astype(np.float64), 1e-6), ang)
            y = y_gpu[0, h, torch.from_numpy(toks).cuda()].float().cpu().numpy().astype(np.float64)
            ratio = np.abs(y - y_ref) / (2.0 ** -8 * np.abs(y_ref) + 1e-5)
            worst = max(worst, float(ratio.max()))
            assert (ratio <= 1.0).all(), (h, float(ratio.max()))
    say(f"  Q/K sampled: worst error / bound {worst:.3f}")
    # 2. the workspace equals sa_pool run on the produced Q/K
    ws_pool = api.sa_pool(q, k, v, grid, tau=tau)
    torch.cuda.synchronize()
    assert torch.equal(ws, ws_pool), "producer workspace differs from sa_pool on its own outputs"
    del ws_pool
    # 3. the attention that follows, against the oracle on the produced operands
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, tau=tau, workspace=ws, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    prod = synth.Inputs(wl, q.cpu(), k.cpu(), inp.v)
    del ws, q, k, v
    mask_np = mask.cpu().numpy()
    del mask
    _check_all(prod, mask_np, lambda bh, m: mask_check(prod, bh[0], bh[1], m, tau), o, lse, tau, seed=9)
