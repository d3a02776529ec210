"""GPU parity of the HIP path (through the C ABI) against the CPU oracle at
sizes the oracle finishes in seconds: several query/key tiles, ragged tails,
odd block counts, two virtual-key chunks, and the degenerate cases (one
token, one ragged block, tau = 0, tau = inf, correction off)."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_route_amd import api, synth
from tests.parity import mask_check, output_check, say, to_gpu

pytestmark = pytest.mark.gpu


def _wl(B=1, H=2, T=3, Hg=10, Wg=13, D=128, dtype="bf16", seed=7, n_sink=0):
    return synth.Workload(f"t{T}x{Hg}x{Wg}_d{D}_{dtype}", B, H, T, Hg, Wg, D, dtype, (2.0,), True,
                          seed=seed, n_sink=n_sink)


def _run_case(wl, tau, correction, qblocks=None, heads=None):
    say(f"case {wl.name} B{wl.B} H{wl.H} N{wl.N} tau={tau} corr={correction}")
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    o, lse, kept = api.sa_forward(q, k, v, grid, tau=tau, correction=correction, q_scale=qs,
                                  k_scale=ks, want_kept=True)
    mask, kept_r = api.sa_route(q, k, v, grid, tau=tau, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    mask_np = mask.cpu().numpy()
    # routing agreement: the fused kernel keeps exactly what sa_route reports
    assert torch.equal(kept.cpu(), kept_r.cpu())
    assert np.array_equal(kept_r.cpu().numpy(), mask_np.sum(axis=-1))
    stats = []
    for b in range(wl.B):
        for h in range(wl.H):
            if heads is not None and (b, h) not in heads:
                continue
            keep, nband, nflip = mask_check(inp, b, h, mask_np[b, h], tau)
            st = output_check(inp, b, h, o, lse, keep, tau, correction, qblocks=qblocks)
            st.update(band=nband, flipped=nflip, density=float(keep.mean()))
            stats.append(st)
    say("  ", stats[:2])
    return inp, o, lse


@pytest.mark.parametrize("tau", [0.0, 1.0, 2.5, math.inf])
@pytest.mark.parametrize("correction", [True, False])
def test_bf16_several_tiles_ragged(tau, correction):
    _run_case(_wl(), tau, correction)


def test_bf16_d64_odd_block_count():
    _run_case(_wl(B=2, H=1, T=2, Hg=16, Wg=17, D=64), 2.0, True)


@pytest.mark.parametrize("tau", [1.0, 4.0])
def test_bf16_two_virtual_chunks(tau):
    # Nb = 71 > 64: the correction streams two chunks of virtual keys
    _run_case(_wl(B=1, H=1, T=5, Hg=30, Wg=30), tau, True, qblocks=[0, 1, 35, 69, 70])


@pytest.mark.parametrize("grid", [(1, 1, 37), (1, 8, 8), (1, 1, 1), (1, 2, 33)])
def test_bf16_tiny_sequences(grid):
    T, Hg, Wg = grid
    _run_case(_wl(B=1, H=2, T=T, Hg=Hg, Wg=Wg), 1.0, True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("tau,correction", [(0.5, True), (4.0, True), (1.0, False), (math.inf, True)])
def test_f32_path(D, tau, correction):
    _run_case(_wl(B=1, H=2, T=2, Hg=12, Wg=13, D=D, dtype="f32"), tau, correction)


@pytest.mark.parametrize("tau", [1.0, 4.0])
def test_fp8_path(tau):
    _run_case(_wl(B=2, H=1, T=3, Hg=10, Wg=13, dtype="fp8"), tau, True)


def test_sink_tokens():
    _run_case(_wl(B=1, H=2, T=3, Hg=12, Wg=13, n_sink=2), 4.0, True)


def test_deterministic_and_pooled_split():
    wl = _wl(B=1, H=3, T=3, Hg=14, Wg=15)
    say(f"case determinism {wl.name}")
    inp = synth.generate(wl)
    q, k, v, _, _ = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    o1, l1, k1 = api.sa_forward(q, k, v, grid, tau=2.0, want_kept=True)
    o2, l2, k2 = api.sa_forward(q, k, v, grid, tau=2.0, want_kept=True)
    ws = api.sa_pool(q, k, v, grid, tau=2.0)
    o3, l3, k3 = api.sa_forward_pooled(q, k, v, grid, tau=2.0, workspace=ws, want_kept=True)
    torch.cuda.synchronize()
    for a, b in [(o1, o2), (l1, l2), (k1, k2), (o1, o3), (l1, l3), (k1, k3)]:
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("fp8", 128)])
def test_dense_path_and_tau_inf(dtype, D):
    wl = _wl(B=1, H=2, T=2, Hg=11, Wg=13, D=D, dtype=dtype)
    say(f"case dense {wl.name}")
    inp = synth.generate(wl)
    q, k, v, qs, ks = to_gpu(inp)
    grid = (wl.T, wl.Hg, wl.Wg)
    od, ld = api.sa_dense_forward(q, k, v, grid, q_scale=qs, k_scale=ks)
    os_, ls_, _ = api.sa_forward(q, k, v, grid, tau=math.inf, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    for h in range(wl.H):
        output_check(inp, 0, h, od, ld, None, math.inf, False, dense=True)
    # tau = inf keeps every block; the virtual keys are all masked
    assert torch.equal(od, os_) and torch.equal(ld, ls_)


def test_identical_value_rows():
    wl = _wl(B=1, H=2, T=3, Hg=10, Wg=13)
    say("case identical V rows")
    inp = synth.generate(wl)
    row = torch.linspace(-1, 1, wl.D).to(torch.bfloat16)
    inp.v[:] = row
    q, k, v, _, _ = to_gpu(inp)
    o, _, _ = api.sa_forward(q, k, v, (wl.T, wl.Hg, wl.Wg), tau=1.0)
    torch.cuda.synchronize()
    err = (o.float().cpu() - row.float()).abs().max().item()
    assert err <= 2e-2, err


def test_explicit_scale():
    wl = _wl(B=1, H=1, T=3, Hg=10, Wg=13)
    say("case explicit scale")
    inp = synth.generate(wl)
    q, k, v, _, _ = to_gpu(inp)
    s = 0.05
    o, lse, _ = api.sa_forward(q, k, v, (wl.T, wl.Hg, wl.Wg), tau=1.0, scale=s)
    mask, _ = api.sa_route(q, k, v, (wl.T, wl.Hg, wl.Wg), tau=1.0, scale=s)
    torch.cuda.synchronize()
    keep, _, _ = mask_check(inp, 0, 0, mask.cpu().numpy()[0, 0], 1.0, scale=s)
    output_check(inp, 0, 0, o, lse, keep, 1.0, True, scale=s)


def test_empty_batch():
    q = torch.empty((0, 2, 64, 128), dtype=torch.bfloat16, device="cuda:0")
    o, lse, _ = api.sa_forward(q, q, q, (1, 8, 8), tau=1.0)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 64, 128) and lse.shape == (0, 2, 64)


def test_maximum_sequence_length():
    # N = SA_MAX_N = 262,144 tokens (Nb = 4096 = the on-chip routing limit)
    wl = _wl(B=1, H=1, T=64, Hg=64, Wg=64)
    assert wl.N == api.MAX_N
    _run_case(wl, 2.0, True, qblocks=[0, 2047, 4094, 4095])
