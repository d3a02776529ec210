"""Pins of the oracle's 3-D tile token order (CPU only).

Blocks formed over the tokens in tile order are cubes of the video token grid
(the Sol-Engine README, section "Sol-Attention", replaces video-token
self-attention; the grid comes with the call).  Expected values come from
hand-written orders (tests/golden/tile_orders.json), an independent
formulation of the order as a sort, the pure-Python brute force of
test_oracle_pins, library routines in special cases, and invariants.
"""
import json
import os

import numpy as np
import pytest

from oracle import attention as orc
from tests import test_oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tile_orders.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c['grid']}-{c['tile']}")
def test_hand_written_orders(case):
    assert orc.tile_order(*case["grid"], case["tile"]).tolist() == case["order"]


def _order_by_sort(T, Hg, Wg, tile):
    # the same order stated as a sort key: tokens of full tiles first, by
    # (tile index, index inside the tile); the rest after them by raster index
    tt, th, tw = tile
    nz, ny, nx = T // tt, Hg // th, Wg // tw

    def key(n):
        t, rem = divmod(n, Hg * Wg)
        y, x = divmod(rem, Wg)
        if t < nz * tt and y < ny * th and x < nx * tw:
            tile_id = ((t // tt) * ny + y // th) * nx + x // tw
            inner = ((t % tt) * th + y % th) * tw + x % tw
            return (0, tile_id, inner)
        return (1, n, 0)
    return sorted(range(T * Hg * Wg), key=key)


@pytest.mark.parametrize("grid", [(21, 45, 80), (3, 10, 13), (4, 16, 16), (2, 7, 9), (1, 1, 37), (5, 3, 3)])
@pytest.mark.parametrize("tile", [(4, 4, 4), (1, 8, 8), (2, 4, 8), (1, 1, 64), (16, 2, 2)])
def test_order_is_the_sorted_tile_order(grid, tile):
    order = orc.tile_order(*grid, tile)
    assert order.tolist() == _order_by_sort(*grid, tile)
    assert np.array_equal(np.sort(order), np.arange(np.prod(grid)))


def test_single_row_tiles_on_a_64_wide_grid_are_the_raster_order():
    assert np.array_equal(orc.tile_order(3, 5, 64, (1, 1, 64)), np.arange(3 * 5 * 64))


def test_dense_limit_is_order_free():
    q, k, v = pins._rand_qkv(4, N=2 * 9 * 16, D=8)
    order = orc.tile_order(2, 9, 16, (2, 4, 8))
    o, lse, _ = orc.forward_head(q, k, v, 64, order=order)
    o_ref, lse_ref = orc.dense_head(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tau", [0.0, 1.0])
def test_tile_constant_kv_is_exact(tau):
    # K and V constant on every block of the tiled order: the n_J copies of a
    # skipped block are then exact, so the output is dense attention on the
    # original token order -- which pins that outputs are scattered back by
    # the same permutation that formed the blocks
    T, Hg, Wg, tile = 3, 10, 13, (1, 8, 8)
    N = T * Hg * Wg
    order = orc.tile_order(T, Hg, Wg, tile)
    rng = np.random.default_rng(8)
    nb = (N + 63) // 64
    kb, vb = rng.normal(size=(nb, 5)) * 2, rng.normal(size=(nb, 5))
    k = np.empty((N, 5))
    v = np.empty((N, 5))
    pos_block = np.arange(N) // 64
    k[order] = kb[pos_block]
    v[order] = vb[pos_block]
    q = rng.normal(size=(N, 5))
    o, lse, keep = orc.forward_head(q, k, v, 64, tau, True, order=order)
    assert not keep.all()                      # some blocks really are skipped
    o_ref, lse_ref = pins._sdpa(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tau,topk", [(0.5, None), (None, 2)])
@pytest.mark.parametrize("corr", [True, False])
def test_brute_force_over_tiled_blocks(tau, topk, corr):
    # brute force on the permuted tokens, scattered back by hand
    T, Hg, Wg, tile = 2, 3, 4, (1, 2, 2)        # 24 tokens, blocks of 4 = 2x2 tiles
    order = orc.tile_order(T, Hg, Wg, tile).tolist()
    rng = np.random.default_rng(13)
    N, D = T * Hg * Wg, 3
    q, k, v = (rng.normal(size=(N, D)) * 1.5 for _ in range(3))
    o, lse, _ = orc.forward_head(q, k, v, 4, 0.0 if tau is None else tau, corr, order=order, topk=topk)
    qp = [q[order[i]].tolist() for i in range(N)]
    kp = [k[order[i]].tolist() for i in range(N)]
    vp = [v[order[i]].tolist() for i in range(N)]
    ob, lb = pins._brute(qp, kp, vp, 4, 0.0 if tau is None else tau, corr, None, topk=topk)
    for i in range(N):
        np.testing.assert_allclose(o[order[i]], ob[i], rtol=1e-12, atol=1e-12)
        assert abs(lse[order[i]] - lb[i]) < 1e-12


def test_invalid_tile_rejected():
    with pytest.raises(ValueError):
        orc.tile_order(2, 2, 2, (0, 1, 1))
