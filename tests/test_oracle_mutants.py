"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies the oracle's source, plants one plausible mistake (a wrong
multiplicity, a pooled instead of per-row correction logit, an exclusive
threshold, a transposed proxy, ...), loads the mutant as a module and checks
that the pins of tests/test_oracle_pins.py reject it.  The unmutated source
must pass the same checks.
"""
import importlib.util
import math
import os
import types

import numpy as np
import pytest

from tests import test_oracle_pins as pins
from tests import test_oracle_tiles as tile_pins
from tests import test_oracle_topk as topk_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "multiplicity_is_block_size": (
        "nJ = np.array([ranges[J][1] - ranges[J][0] for J in skipped], dtype=np.float64)",
        "nJ = np.array([float(block) for J in skipped], dtype=np.float64)"),
    "pooled_correction_logit": (
        "c = s * (q_rows @ kbar.T)",
        "c = np.repeat(s * (q_rows.mean(axis=0, keepdims=True) @ kbar.T), q_rows.shape[0], axis=0)"),
    "exclusive_threshold": ("keep = p >= (m - tau)[:, None]", "keep = p > (m - tau)[:, None]"),
    "threshold_sign": ("keep = p >= (m - tau)[:, None]", "keep = p >= (m + tau)[:, None] - 2 * tau * (tau == np.inf)"),
    "transposed_proxy": ("return s * (qb @ kb.T)", "return s * (kb @ qb.T)"),
    "mean_over_block_size": ("out[J] = x[s:e].sum(axis=0) / (e - s)", "out[J] = x[s:e].sum(axis=0) / block"),
    "lse_drops_max": ("lse = M[:, 0] + np.log(Z[:, 0])", "lse = np.log(Z[:, 0])"),
    "multiplicity_dropped": ("w = weights_mult[None, :] * np.exp(logits - M)", "w = np.exp(logits - M)"),
    "scale_one_over_d": ("return 1.0 / math.sqrt(D)", "return 1.0 / D"),
    "correction_value_is_key_mean": (
        "vbar = np.stack([v[slice(*ranges[J])].mean(axis=0) for J in skipped])",
        "vbar = np.stack([v[slice(*ranges[J])][0] for J in skipped])"),
    "topk_ties_to_larger_index": (
        "order = np.lexsort((np.arange(nb), -p[I]))", "order = np.lexsort((-np.arange(nb), -p[I]))"),
    "topk_smallest_proxies": (
        "order = np.lexsort((np.arange(nb), -p[I]))", "order = np.lexsort((np.arange(nb), p[I]))"),
    "topk_one_short": ("keep[I, order[:kk]] = True", "keep[I, order[:max(kk - 1, 1)]] = True"),
    "tile_inner_order_transposed": (
        "t, y, x = fz * tt + dz, fy * th + dy, fx * tw + dx",
        "t, y, x = fz * tt + (dx % tt), fy * th + dy, fx * tw + (dz % tw)"),
    "tile_leftovers_dropped_to_raster": (
        "if t >= nz * tt or y >= ny * th or x >= nx * tw:",
        "if t >= nz * tt and y >= ny * th and x >= nx * tw:"),
    "tile_outputs_not_scattered_back": ("        o[order] = o_p\n", "        o[:] = o_p[order]\n"),
}


def _load(src: str) -> types.ModuleType:
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    saved = pins.orc
    pins.orc = mod
    try:
        for case in pins._golden_cases():
            for corr in (True, False):
                pins.test_hand_cases_closed_form(case, corr)
        for N, block, D in [(12, 4, 3), (13, 4, 2)]:
            for tau in (0.0, 0.5, math.inf):
                for corr in (True, False):
                    pins.test_brute_force_tiny(N, block, D, tau, corr)
        pins.test_block_constant_kv_is_exact(1.0, 200)
        pins.test_keep_all_equals_sdpa(True)
        topk_pins.orc = mod
        for case in topk_pins._cases():
            topk_pins.test_topk_hand_cases_closed_form(case, True)
        topk_pins.test_topk_brute_force_with_ties()
        for topk in (1, 2, 3):
            topk_pins.test_topk_brute_force_tiny(12, 4, 3, topk, True)
        tile_pins.orc = mod
        for case in tile_pins._cases():
            tile_pins.test_hand_written_orders(case)
        tile_pins.test_tile_constant_kv_is_exact(0.0)
        tile_pins.test_brute_force_over_tiled_blocks(0.5, None, True)
        return True
    except AssertionError:
        return False
    finally:
        pins.orc = saved
        topk_pins.orc = saved
        tile_pins.orc = saved


def _source() -> str:
    with open(SRC) as f:
        return f.read()


def test_unmutated_oracle_passes():
    assert _pins_pass(_load(_source()))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = _source()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    assert not _pins_pass(_load(src.replace(old, new)))
