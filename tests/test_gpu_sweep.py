"""A seeded sweep of GPU parity over the option space (CPU oracle as the
reference): random small grids (ragged and exact block counts), head
dimension, dtype path, threshold or fixed budget, correction off, mean copies
or first order, raster or 3-D tile order, explicit scale, batch and heads.  The draws are fixed by
the seed, so the same cases run every time; each one goes through sa_pool +
sa_forward_pooled, and sa_route for the masks, as the benchmark does."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from oracle import attention as orc
from tests.parity import mask_check, mask_check_topk, output_check, say, to_gpu

pytestmark = pytest.mark.gpu

TILES = [None, (1, 8, 8), (4, 4, 4), (2, 4, 8), (1, 2, 32)]


def _draw(i):
    rng = np.random.default_rng(1000 + i)
    dtype = ["bf16", "bf16", "bf16", "f32", "fp8"][rng.integers(5)]
    D = int(rng.choice([64, 128]))
    T, Hg, Wg = int(rng.integers(1, 5)), int(rng.integers(4, 17)), int(rng.integers(4, 21))
    tile = None if dtype == "fp8" else TILES[rng.integers(len(TILES))]
    if tile is not None and (tile[0] > T or tile[1] > Hg or tile[2] > Wg):
        tile = None
    topk = int(rng.integers(1, 6)) if rng.random() < 0.4 else 0
    tau = float(rng.choice([0.0, 0.5, 1.0, 2.0, 4.0, math.inf])) if not topk else 0.0
    corr = bool(rng.random() < 0.7)
    scale = float(rng.choice([0.0, 0.0, 0.07]))
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    corr = 2 if corr and rng.random() < 0.35 else int(corr)   # 2: the first-order correction
    return dict(dtype=dtype, D=D, grid=(T, Hg, Wg), tile=tile, topk=topk, tau=tau, corr=corr,
                scale=scale, B=B, H=H, seed=2000 + i)


CASES = [_draw(i) for i in range(64)]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_sweep(case):
    T, Hg, Wg = case["grid"]
    wl = synth.Workload(f"sweep{T}x{Hg}x{Wg}", case["B"], case["H"], T, Hg, Wg, case["D"], case["dtype"],
                        (1.0,), case["corr"], seed=case["seed"])
    say(f"case {case}")
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    grid = (T, Hg, Wg)
    kw = dict(tau=case["tau"], topk=case["topk"], correction=case["corr"], scale=case["scale"],
              tile=case["tile"], q_scale=qs, k_scale=ks)
    ws = api.sa_pool(q, k, v, grid, **kw)
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, workspace=ws, want_kept=True, **kw)
    rkw = {x: kw[x] for x in ("tau", "topk", "scale", "tile", "q_scale", "k_scale")}
    mask, kept_r = api.sa_route(q, k, v, grid, **rkw)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    mask_np = mask.cpu().numpy()
    order = None if case["tile"] is None else orc.tile_order(T, Hg, Wg, case["tile"])
    scale = case["scale"] if case["scale"] > 0 else None
    for b in range(wl.B):
        for h in range(wl.H):
            if case["topk"]:
                keep, _, _ = mask_check_topk(inp, b, h, mask_np[b, h], case["topk"], scale=scale, order=order)
            else:
                keep, _, _ = mask_check(inp, b, h, mask_np[b, h], case["tau"], scale=scale, order=order)
            output_check(inp, b, h, o, lse, keep, case["tau"], case["corr"], scale=scale, order=order)
