"""Pins of the oracle's first-order correction (correction = 2), CPU only.

The first-order model replaces each skipped block's value by
vbar_J + (s / n_J) sum_j (qbar_I . (k_j - kbar_J)) v_j and keeps its weight
n_J exp(s q_i . kbar_J).  It is pinned here by what the mathematics fixes,
not by retyping it:

* a per-key brute force in pure Python: every skipped key j gets its own
  weight exp(c_iJ) (1 + s qbar_I . d_j) (the expansion itself), with no
  collapsing into a per-block value;
* convergence order: with the query and key deviations from their block
  means scaled by t, the first-order model differs from dense attention by
  O(t^2) and the mean copies by O(t) -- halving t divides the errors by about
  4 and 2 (a dropped term, a wrong sign or factor breaks the 4);
* special cases: keys constant over each block, or queries whose block mean
  is zero, reduce it to the mean copies exactly;
* invariants: the LSE equals the mean copies' (the deviations sum to zero, so
  the denominator is unchanged), and adding a constant vector to every value
  adds it to every output row.

Planted mistakes (test_mutants_fail_the_pins) must each fail one of these.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import attention as orc

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")


def _random_keep(rng, nb, frac=0.5):
    keep = rng.random((nb, nb)) >= frac
    keep[np.arange(nb), np.arange(nb)] = True
    return keep


def _forward(o, q, k, v, keep, corr, scale=None, block=64):
    return o.forward_head(q, k, v, block, math.inf, corr, scale, keep=keep)


# ------------------------------------------------------------------- pins
def pin_brute_force(o, N=13, block=4, D=3, seed=0):
    """Per-key weights exp(c_iJ) (1 + s qbar_I . d_j) in pure-Python loops."""
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(N, D))
    k = rng.normal(size=(N, D))
    v = rng.normal(size=(N, 2))
    nb = (N + block - 1) // block
    keep = _random_keep(rng, nb)
    s = 0.7
    got, lse, _ = _forward(o, q, k, v, keep, 2, scale=s, block=block)
    blocks = [list(range(b * block, min(N, b * block + block))) for b in range(nb)]
    for I in range(nb):
        qbar = [sum(q[i][d] for i in blocks[I]) / len(blocks[I]) for d in range(D)]
        for i in blocks[I]:
            terms = []  # (log of the positive part of a weight or None, weight factor, value row)
            for J in range(nb):
                if keep[I][J]:
                    for j in blocks[J]:
                        terms.append((s * sum(q[i][d] * k[j][d] for d in range(D)), 1.0, v[j]))
                else:
                    kbar = [sum(k[j][d] for j in blocks[J]) / len(blocks[J]) for d in range(D)]
                    c = s * sum(q[i][d] * kbar[d] for d in range(D))
                    for j in blocks[J]:
                        lin = 1.0 + s * sum(qbar[d] * (k[j][d] - kbar[d]) for d in range(D))
                        terms.append((c, lin, v[j]))
            m = max(t[0] for t in terms)
            num = [0.0, 0.0]
            den = 0.0
            for lg, f, val in terms:
                w = math.exp(lg - m) * f
                den += w
                num[0] += w * val[0]
                num[1] += w * val[1]
            assert abs(got[i][0] - num[0] / den) < 1e-12 and abs(got[i][1] - num[1] / den) < 1e-12
            assert abs(lse[i] - (m + math.log(den))) < 1e-12


def _deviation_case(t, seed=4, N=200, D=16, block=64):
    """q = q0 + t e, k = kbar0 + t d with the deviations centred per block."""
    rng = np.random.default_rng(seed)
    nb = (N + block - 1) // block
    rows = [np.arange(b * block, min(N, b * block + block)) for b in range(nb)]
    q0 = rng.normal(size=(nb, D)) * 2
    k0 = rng.normal(size=(nb, D)) * 2
    e = rng.normal(size=(N, D))
    d = rng.normal(size=(N, D))
    q = np.empty((N, D))
    k = np.empty((N, D))
    for b, r in enumerate(rows):
        q[r] = q0[b] + t * (e[r] - e[r].mean(axis=0))
        k[r] = k0[b] + t * (d[r] - d[r].mean(axis=0))
    v = rng.normal(size=(N, D))
    keep = _random_keep(rng, nb, frac=0.6)
    return q, k, v, keep


def pin_convergence_order(o):
    """Errors against dense attention shrink like t^2 (first order) and t (mean copies)."""
    errs = {1: [], 2: []}
    for t in (2e-2, 1e-2, 5e-3):
        q, k, v, keep = _deviation_case(t)
        ref, _ = o.dense_head(q, k, v)
        for corr in (1, 2):
            got, _, _ = _forward(o, q, k, v, keep, corr)
            errs[corr].append(np.abs(got - ref).max())
    for corr, lo, hi in ((2, 3.6, 4.4), (1, 1.8, 2.2)):
        e = errs[corr]
        for a, b in zip(e, e[1:]):
            assert lo < a / b < hi, (corr, e)
    assert errs[2][-1] < 0.1 * errs[1][-1], errs


def pin_constant_keys(o):
    """Keys constant over each block: no deviation, the mean copies exactly."""
    rng = np.random.default_rng(5)
    N, D, block = 200, 8, 64
    nb = (N + block - 1) // block
    k = np.repeat(rng.normal(size=(nb, D)), block, axis=0)[:N]
    q = rng.normal(size=(N, D))
    v = rng.normal(size=(N, D))
    keep = _random_keep(rng, nb)
    a, la, _ = _forward(o, q, k, v, keep, 1)
    b, lb, _ = _forward(o, q, k, v, keep, 2)
    assert np.abs(a - b).max() < 1e-13 and np.abs(la - lb).max() < 1e-13


def pin_zero_query_mean(o):
    """Queries in +/- pairs inside every block (qbar_I = 0): the mean copies exactly."""
    rng = np.random.default_rng(6)
    N, D, block = 200, 8, 64
    nb = (N + block - 1) // block
    half = rng.normal(size=(N // 2, D))
    q = np.empty((N, D))
    q[0::2], q[1::2] = half, -half          # every block starts at an even row and has even size
    k = rng.normal(size=(N, D)) * 2
    v = rng.normal(size=(N, D))
    keep = _random_keep(rng, nb)
    a, _, _ = _forward(o, q, k, v, keep, 1)
    b, _, _ = _forward(o, q, k, v, keep, 2)
    assert np.abs(a - b).max() < 1e-13


def pin_lse_unchanged(o):
    """Random case: same LSE as the mean copies, different O."""
    rng = np.random.default_rng(7)
    N, D = 300, 16
    q, k, v = (rng.normal(size=(N, D)) * 1.5 for _ in range(3))
    a, la, keep = o.forward_head(q, k, v, 64, 0.0, 1)
    b, lb, keep2 = o.forward_head(q, k, v, 64, 0.0, 2)
    assert (keep == keep2).all() and not keep.all()
    assert np.abs(la - lb).max() < 1e-12
    assert np.abs(a - b).max() > 1e-3


def pin_value_shift(o):
    """O(V + c) = O(V) + c: the first-order weights of a block sum to zero."""
    rng = np.random.default_rng(8)
    N, D = 200, 8
    q, k, v = (rng.normal(size=(N, D)) * 2 for _ in range(3))
    c = rng.normal(size=D) * 5
    keep = _random_keep(rng, 4)
    a, _, _ = _forward(o, q, k, v, keep, 2)
    b, _, _ = _forward(o, q, k, v + c, keep, 2)
    assert np.abs(b - (a + c)).max() < 1e-11


PINS = [pin_brute_force, pin_convergence_order, pin_constant_keys, pin_zero_query_mean,
        pin_lse_unchanged, pin_value_shift]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(orc)


def test_taylor_with_tile_order_and_topk():
    """The first-order model composes with the 3-D tile order and the fixed
    budget as the mean copies do: blocks of permuted tokens, O and LSE back in
    token order, only the skipped blocks' values differ."""
    rng = np.random.default_rng(9)
    T, Hg, Wg, D = 2, 8, 12, 16
    N = T * Hg * Wg
    q, k, v = (rng.normal(size=(N, D)) for _ in range(3))
    order = orc.tile_order(T, Hg, Wg, (2, 4, 8))
    a, la, keep = orc.forward_head(q, k, v, 64, math.inf, 2, topk=2, order=order)
    b, lb, keep2 = orc.forward_head(q[order], k[order], v[order], 64, math.inf, 2, topk=2)
    assert (keep == keep2).all()
    assert np.abs(a[order] - b).max() < 1e-13 and np.abs(la[order] - lb).max() < 1e-13


# ---------------------------------------------------------------- mutants
MUTANTS = {
    "sign": ("return vJ.mean(axis=0) + (s * (d @ np", "return vJ.mean(axis=0) - (s * (d @ np"),
    "no_one_over_n": ("@ vJ / kJ.shape[0]", "@ vJ"),
    "uncentred_keys": ("d = kJ - kJ.mean(axis=0)", "d = kJ"),
    "no_scale": ("return vJ.mean(axis=0) + (s * (d @ np", "return vJ.mean(axis=0) + (1 * (d @ np"),
    "first_query_row": ("qbar = q_rows.mean(axis=0)\n            for t, J", "qbar = q_rows[0]\n            for t, J"),
    "mean_over_block_size": ("@ vJ / kJ.shape[0]", "@ vJ / 64"),
}


def _load(src):
    mod = types.ModuleType("oracle_taylor_mutant")
    exec(compile(src, "oracle_taylor_mutant", "exec"), mod.__dict__)
    return mod


def _fails_a_pin(mod):
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            return True
    return False


def test_unmutated_source_passes():
    assert not _fails_a_pin(_load(open(SRC).read()))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_fail_the_pins(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    assert _fails_a_pin(_load(src.replace(old, new))), f"mutant {name} passes every pin"
