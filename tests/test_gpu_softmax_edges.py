"""GPU parity of the online softmax at its edges: a key block whose logits lie
far above every earlier one (the running maximum has to be raised in the
middle of a row, after weights were already accumulated), and logits that
rise block after block (many raises, and weights taken against a maximum that
lags the true one), sparse and dense, with and without the correction of
the skipped blocks, at logits up to about ten times the workloads' scale.
The standard bars apply: the correction logits take the key means in two
bf16 halves, so their accuracy does not depend on the logit scale."""
import math

import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from tests.parity import mask_check, output_check, say, to_gpu

pytestmark = pytest.mark.gpu


def _inputs(scale_of_block, seed=21):
    # 4 x 16 x 16 tokens: 16 key blocks, so a row crosses many tiles
    wl = synth.Workload("edges_4x16x16", 1, 2, 4, 16, 16, 128, "bf16", (2.0,), True, seed=seed)
    inp = synth.generate(wl)
    k = inp.k.float()
    for J in range(wl.Nb):
        k[:, :, 64 * J:64 * J + 64] *= scale_of_block(J)
    inp.k[:] = k.to(torch.bfloat16)
    return wl, inp


def _check(wl, inp, tau, correction):
    q, k, v, _, _ = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    o, lse, kept = api.sa_forward(q, k, v, grid, tau=tau, correction=correction, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau)
    torch.cuda.synchronize()
    assert torch.equal(kept.cpu(), kept_r.cpu())
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    for h in range(wl.H):
        keep, _, _ = mask_check(inp, 0, h, mask.cpu().numpy()[0, h], tau)
        st = output_check(inp, 0, h, o, lse, keep, tau, correction)
        say("  ", h, st)
    return lse


@pytest.mark.parametrize("tau,correction", [(2.0, True), (2.0, False), (math.inf, False)])
def test_late_dominant_block(tau, correction):
    # block 11's keys scaled 10x: logits up to ~100 natural units, far more
    # than 64 in log2 units above what the row has seen before
    wl, inp = _inputs(lambda J: 10.0 if J == 11 else 1.0)
    say(f"case late dominant block tau={tau} corr={correction}")
    lse = _check(wl, inp, tau, correction)
    assert float(lse.max()) > 64 * math.log(2)      # the case really reaches the raise


@pytest.mark.parametrize("tau,correction", [(2.0, True), (2.0, False), (math.inf, False)])
def test_rising_logits(tau, correction):
    # key blocks scaled 1, 1.8, 2.6, ...: every tile's maximum exceeds the last
    wl, inp = _inputs(lambda J: 1.0 + 0.8 * J)
    say(f"case rising logits tau={tau} corr={correction}")
    _check(wl, inp, tau, correction)


def test_dense_kernel_late_dominant_block():
    wl, inp = _inputs(lambda J: 10.0 if J == 11 else 1.0)
    say("case dense kernel, late dominant block")
    q, k, v, _, _ = to_gpu(inp)
    od, ld = api.sa_dense_forward(q, k, v, (wl.T, wl.Hg, wl.Wg))
    torch.cuda.synchronize()
    for h in range(wl.H):
        output_check(inp, 0, h, od, ld, None, math.inf, False, dense=True)
