"""GPU parity of the dense path (sa_dense_forward, the tau = inf limit and the
"Dense" baseline of the Sol-Attn page's speedup strip) at full workload size,
in the launch configuration the benchmark times: the 720p shape (B1 H40
N75,600 D128 bf16, 11,840 workgroups, so the XCD-aware tile remap is active)
and the 720p CFG shape with fp8 Q/K (B2 H40, 23,680 workgroups).

Outputs are sampled where the oracle computes them one row block at a time:
heads (0,0), (B-1,H-1) and two seeded random heads, each at its first, ragged
last and two random query blocks, against the float64 dense softmax
attention on the same (bf16-rounded or dequantised) inputs, at the bf16 and
fp8 bars."""
import numpy as np
import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from tests.parity import output_check, say, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["720p", "720p_cfg_fp8"])
def test_dense_full_size(name):
    wl = synth.workload(name)
    say(f"case dense {name}: B{wl.B} H{wl.H} N{wl.N} D{wl.D} {wl.dtype}")
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    o, lse = api.sa_dense_forward(q, k, v, grid, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    del q, k, v
    rng = np.random.default_rng(321)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    sample = {(0, 0), (wl.B - 1, wl.H - 1)}
    while len(sample) < 4:
        sample.add(heads[int(rng.integers(len(heads)))])
    for (b, h) in sorted(sample):
        qb = {0, wl.Nb - 1, int(rng.integers(wl.Nb)), int(rng.integers(wl.Nb))}
        st = output_check(inp, b, h, o, lse, None, float("inf"), False, qblocks=qb, dense=True)
        say(f"  head ({b},{h}) blocks {sorted(qb)}: {st}")
