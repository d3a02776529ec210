"""sa_forward_noalloc (the workspace in the library's static device scratch)
against sa_forward with a caller workspace, through the C ABI, on calls in a
row whose inputs shrink: the same kernels on the same inputs, so the outputs
must agree bit for bit -- the scratch keeps the previous call's contents, and
every call must rewrite all that it reads."""
import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from tests.parity import say, to_gpu

pytestmark = pytest.mark.gpu


def _both(wl, tau, corr=1, topk=0, tile=None):
    say(f"case noalloc {wl.name} B{wl.B} H{wl.H} N{wl.N} {wl.dtype} tau={tau} corr={corr} topk={topk} tile={tile}")
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    kw = dict(tau=tau, correction=corr, topk=topk, tile=tile, q_scale=qs, k_scale=ks, want_kept=True)
    o2, l2, k2 = api.sa_forward_noalloc(q, k, v, grid, **kw)
    o1, l1, k1 = api.sa_forward(q, k, v, grid, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "O differs between sa_forward and sa_forward_noalloc"
    assert torch.equal(l1, l2), "LSE differs"
    assert torch.equal(k1, k2), "kept counts differ"


def test_noalloc_two_calls_second_smaller():
    # Nb = 75 (two chunks of correction tiles, ragged tail), then a 5-block case
    big = synth.Workload("noalloc_big", 1, 4, 4, 30, 40, 128, "bf16", (2.0,), True, seed=61)
    small = synth.Workload("noalloc_small", 1, 2, 2, 10, 13, 128, "bf16", (2.0,), True, seed=62)
    _both(big, 2.0)
    _both(small, 1.0)


def test_noalloc_options_shrinking():
    # fp8 Q/K, then the first-order correction in a 3-D tile order, then a
    # fixed budget at D = 64: each smaller than the one before
    _both(synth.Workload("noalloc_fp8", 2, 2, 3, 20, 24, 128, "fp8", (2.0,), True, seed=63), 2.0)
    _both(synth.Workload("noalloc_first_order", 1, 2, 4, 8, 20, 128, "bf16", (1.0,), True, seed=64), 1.0,
          corr=2, tile=(2, 4, 8))
    _both(synth.Workload("noalloc_topk", 1, 1, 2, 9, 14, 64, "bf16", (0.0,), True, seed=65), 0.0, topk=2)
