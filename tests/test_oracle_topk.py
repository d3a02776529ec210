"""Pins of the oracle's fixed-budget routing (CPU only).

Fixed-budget routing keeps, per query block, the topk key blocks with the
largest pooled proxy, equal proxies in increasing block order (paper review of
the Sol Video Inference Engine, xllm-io blog: PISA at block size 64 and a fixed
sparsity).  Expected values come from hand-derived closed forms
(tests/golden/topk_cases.json), the pure-Python brute force of
test_oracle_pins, library routines in special cases, and invariants.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as orc
from tests import test_oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topk_cases.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("corr", [True, False])
def test_topk_hand_cases_closed_form(case, corr):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k"], dtype=np.float64)
    v = np.array(case["v"], dtype=np.float64)
    keep, _, _ = orc.route_topk(q, k, case["block"], case["topk"], case["scale"])
    assert keep.astype(int).tolist() == case["keep"]
    o, lse, _ = orc.forward_head(q, k, v, case["block"], correction=corr, scale=case["scale"],
                                 topk=case["topk"])
    exp_block = case["correction_on" if corr else "correction_off"]
    o_ref = np.array([[pins._eval(e) for e in row] for row in exp_block["o"]])
    lse_ref = np.array([pins._eval(e) for e in exp_block["lse"]])
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("N,block,D", [(7, 2, 1), (12, 4, 3), (16, 4, 5), (13, 4, 2), (9, 3, 4)])
@pytest.mark.parametrize("topk", [1, 2, 3, 100])
@pytest.mark.parametrize("corr", [True, False])
def test_topk_brute_force_tiny(N, block, D, topk, corr):
    rng = np.random.default_rng(7000 + 1000 * N + 10 * D + block)
    q = rng.normal(size=(N, D)) * 1.5
    k = rng.normal(size=(N, D)) * 1.5
    v = rng.normal(size=(N, D + 1))
    o, lse, _ = orc.forward_head(q, k, v, block, correction=corr, topk=topk)
    nb = (N + block - 1) // block
    ob, lb = pins._brute(q.tolist(), k.tolist(), v.tolist(), block, 0.0, corr, None, topk=min(topk, nb))
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12, atol=1e-12)


def test_topk_brute_force_with_ties():
    # duplicated key blocks give exactly equal proxies: the smaller index wins
    rng = np.random.default_rng(5)
    base = rng.normal(size=(4, 3))
    k = np.concatenate([base, rng.normal(size=(4, 3)), base, base])   # blocks 0, 2, 3 identical
    q = rng.normal(size=(16, 3))
    v = rng.normal(size=(16, 2))
    for topk in (1, 2, 3):
        keep, p, _ = orc.route_topk(q, k, 4, topk)
        assert p[0, 0] == p[0, 2] == p[0, 3]
        o, lse, _ = orc.forward_head(q, k, v, 4, topk=topk)
        ob, lb = pins._brute(q.tolist(), k.tolist(), v.tolist(), 4, 0.0, True, None, topk=topk)
        np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12, atol=1e-12)


def test_topk_counts_nesting_and_level_set():
    q, k, _ = pins._rand_qkv(11, N=300, D=8)
    nb = (300 + 63) // 64
    prev = None
    for topk in range(1, nb + 3):
        keep, p, pk = orc.route_topk(q, k, 64, topk)
        assert (keep.sum(axis=1) == min(topk, nb)).all()
        # with distinct proxies the kept set is the level set p >= k-th largest
        np.testing.assert_array_equal(keep, p >= pk[:, None])
        if prev is not None:
            assert (keep >= prev).all()          # kept(k) contains kept(k - 1)
        prev = keep
    # top-1 is the argmax, i.e. threshold routing at tau = 0 when the max is unique
    keep1, _, _ = orc.route_topk(q, k, 64, 1)
    keep0, _, _ = orc.route(q, k, 64, 0.0)
    np.testing.assert_array_equal(keep1, keep0)


@pytest.mark.parametrize("corr", [True, False])
def test_topk_all_blocks_equals_sdpa(corr):
    q, k, v = pins._rand_qkv(3, N=200, D=16)
    o, lse, _ = orc.forward_head(q, k, v, 64, correction=corr, topk=10 ** 6)
    o_ref, lse_ref = pins._sdpa(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("topk", [1, 2])
def test_topk_block_constant_kv_is_exact(topk):
    # block-constant K and V make every skipped block's n_J copies exact
    rng = np.random.default_rng(21)
    N, D = 200, 6
    kb = rng.normal(size=(4, D)) * 2
    vb = rng.normal(size=(4, D))
    k = np.repeat(kb, 64, axis=0)[:N]
    v = np.repeat(vb, 64, axis=0)[:N]
    q = rng.normal(size=(N, D))
    o, lse, _ = orc.forward_head(q, k, v, 64, correction=True, topk=topk)
    o_ref, lse_ref = pins._sdpa(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("topk", [0, -3])
def test_invalid_topk_rejected(topk):
    q, k, _ = pins._rand_qkv(1, N=64, D=4)
    with pytest.raises(ValueError):
        orc.route_topk(q, k, 64, topk)


def test_batched_topk_matches_heads():
    rng = np.random.default_rng(9)
    q = rng.normal(size=(2, 2, 130, 4))
    k = rng.normal(size=(2, 2, 130, 4))
    v = rng.normal(size=(2, 2, 130, 4))
    o, lse, keep = orc.forward(q, k, v, 64, topk=2)
    for b in range(2):
        for h in range(2):
            oh, lh, kh = orc.forward_head(q[b, h], k[b, h], v[b, h], 64, topk=2)
            np.testing.assert_array_equal(o[b, h], oh)
            np.testing.assert_array_equal(lse[b, h], lh)
            np.testing.assert_array_equal(keep[b, h], kh)
            assert not math.isnan(float(o[b, h].sum()))
