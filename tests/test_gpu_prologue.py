"""GPU parity of the fused Q/K producer step (per-head RMS norm with gain,
3-D rotary embedding, bf16 rounding, pooling) through the C ABI: its Q/K
against the CPU oracle, its workspace bit for bit against sa_pool run on its
own outputs, and the attention that follows against the oracle; raster and
3-D tile order, D 64 and 128, in place."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from oracle import attention as orc
from oracle import prologue as pro
from tests.parity import mask_check, output_check, say

pytestmark = pytest.mark.gpu


def _case(T, Hg, Wg, D, H=2, seed=3):
    wl = synth.Workload(f"p{T}x{Hg}x{Wg}_d{D}", 1, H, T, Hg, Wg, D, "bf16", (1.0,), True, seed=seed)
    inp = synth.generate(wl)     # raw projections: the smooth fields, before norm and rotation
    rng = np.random.default_rng(seed)
    gq = torch.from_numpy(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    gk = torch.from_numpy(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    return wl, inp, gq, gk


def _run(T, Hg, Wg, D, tile=None, in_place=False, tau=1.0, eps=1e-6, base=10000.0):
    wl, inp, gq, gk = _case(T, Hg, Wg, D)
    say(f"case {wl.name} tile={tile} in_place={in_place}")
    dev = torch.device("cuda:0")
    xq, xk, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    grid = (T, Hg, Wg)
    qo = xq.clone() if in_place else None
    ko = xk.clone() if in_place else None
    src_q, src_k = (qo, ko) if in_place else (xq, xk)
    q, k, ws = api.sa_qk_prologue(src_q, src_k, v, grid, gq.to(dev), gk.to(dev), norm_eps=eps, rope_base=base,
                                  tau=tau, tile=tile, q_out=qo, k_out=ko)
    torch.cuda.synchronize()
    order = None if tile is None else orc.tile_order(T, Hg, Wg, tile)
    # 1. Q/K against the oracle (one bf16 rounding of a float32 result)
    for h in range(wl.H):
        for x_raw, g, y_gpu in ((inp.q, gq, q), (inp.k, gk, k)):
            x = x_raw[0, h].to(torch.float64).numpy()
            y_ref = pro.apply_rope(pro.rms_norm(x, g.numpy().astype(np.float64), eps),
                                   pro.rope_angles(T, Hg, Wg, D, base))
            yg = y_gpu[0, h].float().cpu().numpy().astype(np.float64)
            err = np.abs(yg - y_ref)
            bound = 2.0 ** -8 * np.abs(y_ref) + 1e-5
            assert (err <= bound).all(), (h, float(err.max()), float((err / bound).max()))
    # 2. the workspace equals sa_pool run on the produced Q/K
    ws_pool = api.sa_pool(q, k, v, grid, tau=tau, tile=tile)
    torch.cuda.synchronize()
    assert torch.equal(ws, ws_pool), "producer workspace differs from sa_pool on its own outputs"
    # 3. the attention that follows, against the oracle on the produced operands
    o, lse, kept = api.sa_forward_pooled(q, k, v, grid, tau=tau, tile=tile, workspace=ws, want_kept=True)
    mask, _ = api.sa_route(q, k, v, grid, tau=tau, tile=tile)
    torch.cuda.synchronize()
    prod = synth.Inputs(wl, q.cpu(), k.cpu(), v.cpu())
    for h in range(wl.H):
        keep, nband, nflip = mask_check(prod, 0, h, mask.cpu().numpy()[0, h], tau, order=order)
        st = output_check(prod, 0, h, o, lse, keep, tau, True, order=order)
        say("  ", h, st, nband, nflip)


@pytest.mark.parametrize("D", [128, 64])
def test_raster_order(D):
    _run(3, 10, 13, D)


def test_tile_order_and_ragged_grid():
    _run(5, 12, 19, 128, tile=(4, 4, 4))


def test_in_place():
    _run(2, 8, 9, 128, in_place=True)


def test_other_base_and_eps():
    _run(2, 9, 10, 128, eps=1e-3, base=500.0)


def test_rejects_non_bf16():
    wl = synth.Workload("p32", 1, 1, 1, 8, 8, 64, "f32", (1.0,), True, seed=1)
    inp = synth.generate(wl)
    dev = torch.device("cuda:0")
    g = torch.ones(64, device=dev)
    with pytest.raises(api.SaError) as e:
        api.sa_qk_prologue(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), (1, 8, 8), g, g)
    assert e.value.status == 7


def test_batch_and_heads_past_one_workgroup():
    # B = 2, H = 5: ten (b, h) heads, more than the eight that one producer
    # workgroup takes, so the second workgroup row holds only two
    B, H, T, Hg, Wg, D = 2, 5, 2, 8, 9, 128
    wl = synth.Workload(f"pb{B}h{H}", B, H, T, Hg, Wg, D, "bf16", (1.0,), True, seed=5)
    say(f"case {wl.name}")
    inp = synth.generate(wl)
    rng = np.random.default_rng(5)
    gq = torch.from_numpy(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    gk = torch.from_numpy(rng.uniform(0.5, 1.5, size=D).astype(np.float32))
    dev = torch.device("cuda:0")
    xq, xk, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    grid = (T, Hg, Wg)
    q, k, ws = api.sa_qk_prologue(xq, xk, v, grid, gq.to(dev), gk.to(dev), tau=1.0)
    torch.cuda.synchronize()
    ang = pro.rope_angles(T, Hg, Wg, D, 10000.0)
    for b in range(B):
        for h in range(H):
            for x_raw, g, y_gpu in ((inp.q, gq, q), (inp.k, gk, k)):
                x = x_raw[b, h].to(torch.float64).numpy()
                y_ref = pro.apply_rope(pro.rms_norm(x, g.numpy().astype(np.float64), 1e-6), ang)
                yg = y_gpu[b, h].float().cpu().numpy().astype(np.float64)
                assert (np.abs(yg - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-5).all(), (b, h)
    ws_pool = api.sa_pool(q, k, v, grid, tau=1.0)
    torch.cuda.synchronize()
    assert torch.equal(ws, ws_pool)
