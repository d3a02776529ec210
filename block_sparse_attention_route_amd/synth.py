"""Seeded synthetic video-DiT attention inputs (shared by tests, bench and smoke).

This module holds only input generation: smooth random fields over the video
token grid, dtype casts and the per-block fp8 quantisation of the inputs.  It
contains none of the attention method's arithmetic, and both the HIP library
and the CPU oracle receive exactly the arrays it returns.

No page gives activations or a public benchmark for this operator, so the
workloads are stand-ins with the pages' shapes: a Wan2.1-T2V-14B-like 720p
grid (21 x 45 x 80 tokens, 720x1280 at 81 frames; Sol-Engine README, "Models
& speedups" and measurement conditions), an 832x480-like grid (21 x 30 x 52)
and an LTX-2.3 1088x1920-like refinement grid (21 x 68 x 120).

Recipe, per (batch b, head h), seeded by numpy SeedSequence([seed, b, h])
spawned into four streams (Q, K, V, scaling):
* token n = (t*Hg + y)*Wg + x (frame-major raster), position
  u = (t/T, y/Hg, x/Wg);
* Q and K independently: sum over s = 1..4 of a_s * sin(2*pi*f_s.u + phi_s)
  plus 0.3 * eps, with f_s ~ U[0, 0.5)^3 cycles per axis extent (the time
  axis may use a smaller maximum), phi_s ~ U[0, 2*pi), a_s and eps ~ N(0, 1)
  per feature;
* Q and K are both multiplied by c = sqrt(3 / std(q_i.k_j / sqrt(D))) over
  65,536 random pairs, which sets the per-head logit std to about 3 (c = 1
  when that std is below 1e-6, e.g. a single-token grid);
* optional sink tokens: rows 0..n_sink-1 of Q and K rescaled to 4x the mean
  row norm of their tensor (after the scaling);
* V ~ N(0, 1);
* cast last: fp32, bf16 (round to nearest even), or fp8 e4m3fn with one fp32
  scale per (b, h, 64-token block): scale = amax / 448 (1 if amax = 0),
  code = RNE(x / scale) clamped to +-448.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "Inputs", "FP8_MAX"]

FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    Hg: int
    Wg: int
    D: int
    dtype: str                 # "f32", "bf16" or "fp8" (fp8 e4m3 Q/K + bf16 V)
    taus: tuple
    correction: bool = True
    seed: int = 0
    n_sink: int = 0
    ft_max: float = 0.5        # maximum time-axis frequency, cycles per extent
    block: int = 64

    @property
    def N(self) -> int:
        return self.T * self.Hg * self.Wg

    @property
    def Nb(self) -> int:
        return (self.N + self.block - 1) // self.block

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 4, 16, 16, 64, "f32", (4.0,), True, seed=0),
    "480p": Workload("480p", 1, 20, 21, 30, 52, 128, "bf16", (4.0,), True, seed=1, n_sink=2),
    "720p": Workload("720p", 1, 40, 21, 45, 80, 128, "bf16", (2.0, 4.0, 8.0), True, seed=2),
    "1080p": Workload("1080p", 1, 32, 21, 68, 120, 128, "bf16", (4.0,), True, seed=3, ft_max=0.25),
    "720p_cfg_fp8": Workload("720p_cfg_fp8", 2, 40, 21, 45, 80, 128, "fp8", (4.0,), True, seed=4),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


@dataclasses.dataclass
class Inputs:
    """Host tensors in the dtype the kernels read, [B, H, N, D] contiguous."""
    wl: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    q_scale: torch.Tensor | None = None   # [B, H, Nb] fp32 (fp8 only)
    k_scale: torch.Tensor | None = None

    def head64(self, b: int, h: int):
        """The exact values the kernels see for one head, as float64 numpy arrays."""
        def deq(x, s):
            xf = x[b, h].to(torch.float64)
            if s is not None:
                rep = torch.repeat_interleave(s[b, h].to(torch.float64), self.wl.block)[: xf.shape[0]]
                xf = xf * rep[:, None]
            return xf.numpy()
        return deq(self.q, self.q_scale), deq(self.k, self.k_scale), deq(self.v, None)


def _field(rng: np.random.Generator, u: np.ndarray, D: int, ft_max: float) -> np.ndarray:
    # Plain elementwise sums in a fixed order, no BLAS: heads are generated in
    # parallel threads, and concurrent multi-threaded BLAS calls from several
    # threads have returned wrong products with this numpy's OpenBLAS.
    N = u.shape[0]
    f = rng.uniform(0.0, 0.5, size=(4, 3))
    f[:, 0] = rng.uniform(0.0, ft_max, size=4)
    phi = rng.uniform(0.0, 2 * math.pi, size=4)
    a = rng.standard_normal(size=(4, D))
    arg = u[:, 0:1] * f[None, :, 0] + u[:, 1:2] * f[None, :, 1] + u[:, 2:3] * f[None, :, 2]   # [N, 4]
    waves = np.sin(2 * math.pi * arg + phi[None, :])
    x = waves[:, 0:1] * a[0]
    for s in range(1, 4):
        x += waves[:, s:s + 1] * a[s]
    x = x.astype(np.float32)
    x += np.float32(0.3) * rng.standard_normal(size=(N, D), dtype=np.float32)
    return x


def _positions(T: int, Hg: int, Wg: int) -> np.ndarray:
    t, y, x = np.meshgrid(np.arange(T) / T, np.arange(Hg) / Hg, np.arange(Wg) / Wg, indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)


def _head(wl: Workload, b: int, h: int, u: np.ndarray):
    rq, rk, rv, rs = [np.random.Generator(np.random.PCG64(s))
                      for s in np.random.SeedSequence([wl.seed, b, h]).spawn(4)]
    q = _field(rq, u, wl.D, wl.ft_max)
    k = _field(rk, u, wl.D, wl.ft_max)
    v = rv.standard_normal(size=(wl.N, wl.D), dtype=np.float32)
    i = rs.integers(0, wl.N, size=65536)
    j = rs.integers(0, wl.N, size=65536)
    logit = np.einsum("nd,nd->n", q[i].astype(np.float64), k[j].astype(np.float64)) / math.sqrt(wl.D)
    sd = logit.std()
    # a grid of one token (or identical tokens) has no logit spread to normalise
    c = np.float32(math.sqrt(3.0 / sd) if sd > 1e-6 else 1.0)
    q *= c
    k *= c
    for x in (q, k):
        if wl.n_sink:
            target = 4.0 * np.linalg.norm(x, axis=1).mean()
            for n in range(wl.n_sink):
                x[n] *= np.float32(target / max(np.linalg.norm(x[n]), 1e-12))
    return q, k, v


def _fp8_quantise(x: torch.Tensor, block: int):
    """Per-64-token-block scale = amax/448 (1 if amax = 0); codes RNE, clamped to +-448."""
    N, D = x.shape
    Nb = (N + block - 1) // block
    pad = Nb * block - N
    xp = torch.nn.functional.pad(x, (0, 0, 0, pad)).view(Nb, block, D)
    amax = xp.abs().amax(dim=(1, 2))
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).to(torch.float32)
    codes = (xp / scale[:, None, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes.view(Nb * block, D)[:N].contiguous(), scale


def generate(wl: Workload, threads: int | None = None) -> Inputs:
    """Generate the seeded inputs of a workload (host tensors)."""
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    u = _positions(wl.T, wl.Hg, wl.Wg)
    qk_dtype = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[wl.dtype]
    v_dtype = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    q = torch.empty((B, H, N, D), dtype=qk_dtype)
    k = torch.empty((B, H, N, D), dtype=qk_dtype)
    v = torch.empty((B, H, N, D), dtype=v_dtype)
    qs = ks = None
    if wl.dtype == "fp8":
        qs = torch.empty((B, H, wl.Nb), dtype=torch.float32)
        ks = torch.empty((B, H, wl.Nb), dtype=torch.float32)

    def one(bh):
        b, h = divmod(bh, H)
        qh, kh, vh = _head(wl, b, h, u)
        v[b, h] = torch.from_numpy(vh).to(v_dtype)
        if wl.dtype == "fp8":
            q[b, h], qs[b, h] = _fp8_quantise(torch.from_numpy(qh), wl.block)
            k[b, h], ks[b, h] = _fp8_quantise(torch.from_numpy(kh), wl.block)
        else:
            q[b, h] = torch.from_numpy(qh).to(qk_dtype)
            k[b, h] = torch.from_numpy(kh).to(qk_dtype)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(B * H)))
    return Inputs(wl, q, k, v, qs, ks)
