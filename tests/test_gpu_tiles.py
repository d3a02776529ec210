"""GPU parity of the 3-D tile token order (blocks are tiles of the video token
grid, uncovered tokens after them in raster order) through the C ABI against
the CPU oracle: masks, kept counts and outputs for tiles with and without
leftover tokens, threshold and fixed-budget routing, bf16 (D 128 and 64) and
fp32, and the dense limit, which the order must not change."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from oracle import attention as orc
from tests.parity import mask_check, mask_check_topk, output_check, say, to_gpu

pytestmark = pytest.mark.gpu


def _wl(B=1, H=2, T=3, Hg=10, Wg=13, D=128, dtype="bf16", seed=17):
    return synth.Workload(f"g{T}x{Hg}x{Wg}_d{D}_{dtype}", B, H, T, Hg, Wg, D, dtype, (1.0,), True, seed=seed)


def _run(wl, tile, tau=1.0, topk=0, correction=True, qblocks=None):
    say(f"case {wl.name} B{wl.B} H{wl.H} N{wl.N} tile={tile} tau={tau} topk={topk} corr={correction}")
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    o, lse, kept = api.sa_forward(q, k, v, grid, tau=tau, topk=topk, correction=correction, tile=tile,
                                  q_scale=qs, k_scale=ks, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau, topk=topk, tile=tile, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    mask_np = mask.cpu().numpy()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    assert np.array_equal(kept_r.cpu().numpy(), mask_np.sum(axis=-1))
    order = orc.tile_order(wl.T, wl.Hg, wl.Wg, tile)
    stats = []
    for b in range(wl.B):
        for h in range(wl.H):
            if topk:
                keep, nband, nflip = mask_check_topk(inp, b, h, mask_np[b, h], topk, order=order)
            else:
                keep, nband, nflip = mask_check(inp, b, h, mask_np[b, h], tau, order=order)
            st = output_check(inp, b, h, o, lse, keep, tau, correction, qblocks=qblocks, order=order)
            st.update(band=nband, flipped=nflip, density=float(keep.mean()))
            stats.append(st)
    say("  ", stats[:2])
    return o, lse


@pytest.mark.parametrize("tile", [(1, 8, 8), (2, 4, 8), (4, 4, 4), (1, 1, 64)])
@pytest.mark.parametrize("correction", [True, False])
def test_bf16_tiles_with_leftovers(tile, correction):
    _run(_wl(T=5, Hg=12, Wg=19), tile, correction=correction)   # every tile leaves tokens over


def test_exact_cover_no_leftovers():
    _run(_wl(T=4, Hg=16, Wg=16), (4, 4, 4), tau=2.0)


@pytest.mark.parametrize("topk", [1, 3])
def test_fixed_budget_in_tile_order(topk):
    _run(_wl(T=5, Hg=12, Wg=19), (1, 8, 8), topk=topk)


def test_d64_bf16():
    _run(_wl(T=4, Hg=9, Wg=17, D=64), (2, 4, 8), tau=0.5)


@pytest.mark.parametrize("D", [64, 128])
def test_f32_path(D):
    _run(_wl(T=3, Hg=9, Wg=10, D=D, dtype="f32"), (1, 8, 8), tau=1.0)


def test_two_virtual_chunks_and_sampled_blocks():
    _run(_wl(H=1, T=8, Hg=24, Wg=30), (4, 4, 4), tau=1.0, qblocks=[0, 1, 50, 63, 64, 88, 89])


def test_order_free_at_tau_inf():
    wl = _wl(T=3, Hg=12, Wg=19)
    o_t, lse_t = _run(wl, (4, 4, 4), tau=math.inf)
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    o_r, lse_r, _ = api.sa_forward(q, k, v, (wl.T, wl.Hg, wl.Wg), tau=math.inf)
    torch.cuda.synchronize()
    assert (o_t.float() - o_r.float()).abs().max().item() <= 2e-2
    assert (lse_t - lse_r).abs().max().item() <= 1e-3


def test_fp8_with_tiles_is_rejected():
    wl = _wl(T=2, Hg=8, Wg=8, dtype="fp8")
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    with pytest.raises(api.SaError) as e:
        api.sa_forward(q, k, v, (wl.T, wl.Hg, wl.Wg), tau=1.0, tile=(4, 4, 4), q_scale=qs, k_scale=ks)
    assert e.value.status == 7        # SA_ERR_UNSUPPORTED


def test_batch_of_two():
    # CFG-like batch: heads (b, h) indexed b * H + h in every tiled buffer
    _run(_wl(B=2, H=2, T=3, Hg=10, Wg=13), (1, 8, 8), tau=1.0)
