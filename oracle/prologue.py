"""Plain CPU oracle for the Q/K producer step that feeds the attention:
per-head RMS normalisation, 3-D rotary position embedding, and the block
means the routing needs.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes
----------------
The paper review of the Sol Video Inference Engine (xllm-io blog, kernel
fusion candidates, and the LTX-2.3 settings) lists a fused RoPE + norm and a
fused QK + RoPE among the lossless fusions in front of attention; the Sol-Attn
project page (section "Abstract") routes on a pooled score of the resulting
Q and K.  The pages give no formula, so the plainest reading is fixed here
(every reading is listed in the design notes of the repository):

* per head and token, RMS normalisation over the D features with a learned
  gain g (shared by the heads): y = x / sqrt(mean(x^2) + eps) * g;
* then rotary embedding over the video grid: the D/2 feature pairs
  (2j, 2j + 1) are split into three consecutive groups for the frame, row and
  column coordinates of the token -- d_t = D - 4 * (D // 6) features for t,
  2 * (D // 6) each for y and x -- and pair j of a group of d_a features is
  rotated by the angle pos_a * base^(-2 j / d_a);
* the results are rounded to bf16 (the attention's operands), and the block
  means of the rounded values are the routing operands qbar, kbar.

Pinned by tests/test_oracle_prologue.py (closed forms, the complex-number
form of the rotation, norm and relative-position invariants).  Parity
unpinned: none.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rope_split", "rms_norm", "rope_angles", "apply_rope", "qk_prologue"]


def rope_split(D: int) -> tuple[int, int, int]:
    """Feature counts (d_t, d_y, d_x) of the three rotary groups."""
    if D % 2 or D < 6:
        raise ValueError("D must be even and at least 6")
    dy = 2 * (D // 6)
    return D - 2 * dy, dy, dy


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean over features of x^2 + eps) * gain, row by row."""
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def rope_angles(T: int, Hg: int, Wg: int, D: int, base: float) -> np.ndarray:
    """Angle of every (token, pair): [N, D/2], tokens in the raster order."""
    dt, dy, dx = rope_split(D)
    tok = np.arange(T * Hg * Wg)
    pos = (tok // (Hg * Wg), (tok // Wg) % Hg, tok % Wg)
    cols = []
    for d_a, p in zip((dt, dy, dx), pos):
        j = np.arange(d_a // 2)
        theta = base ** (-2.0 * j / d_a)
        cols.append(p[:, None].astype(np.float64) * theta[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate each feature pair (2j, 2j+1) by its angle."""
    x = np.asarray(x, dtype=np.float64)
    a, b = x[..., 0::2], x[..., 1::2]
    c, s = np.cos(angles), np.sin(angles)
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def _bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest even), returned as float64."""
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def qk_prologue(x: np.ndarray, gain: np.ndarray, T: int, Hg: int, Wg: int, base: float = 10000.0,
                eps: float = 1e-6, block: int = 64, order=None):
    """One head: x [N, D] (raw projection, float) -> (y [N, D] rounded to
    bf16 as float64, means [Nb, D] of the rounded y over the blocks of the
    given position order, or of the raster order)."""
    x = np.asarray(x, dtype=np.float64)
    N, D = x.shape
    y = apply_rope(rms_norm(x, gain, eps), rope_angles(T, Hg, Wg, D, base))
    # float64 -> float32 -> bf16: the product path rounds its float32 result once
    yb = _bf16(y)
    pos = yb if order is None else yb[np.asarray(order)]
    nb = (N + block - 1) // block
    means = np.stack([pos[block * J: min(block * J + block, N)].mean(axis=0) for J in range(nb)])
    return yb, means

