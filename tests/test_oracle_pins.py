"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a hand-derived closed form
(tests/golden/hand_cases.json), a pure-Python brute force written from the
definition, a library routine in a special case, or an invariant of the
mathematics.  The definition is the reading of the Sol-Attn project page
(section "Abstract") recorded in the oracle's module docstring.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ----------------------------------------------------------------------------
# hand-derived closed forms
# ----------------------------------------------------------------------------

def _eval(expr):
    return eval(expr, {"__builtins__": {}}, {"exp": math.exp, "log": math.log})


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("corr", [True, False])
def test_hand_cases_closed_form(case, corr):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k"], dtype=np.float64)
    v = np.array(case["v"], dtype=np.float64)
    keep, _, _ = orc.route(q, k, case["block"], case["tau"], case["scale"])
    assert keep.astype(int).tolist() == case["keep"]
    o, lse, _ = orc.forward_head(q, k, v, case["block"], case["tau"], corr, case["scale"])
    exp_block = case["correction_on" if corr else "correction_off"]
    o_ref = np.array([[_eval(e) for e in row] for row in exp_block["o"]])
    lse_ref = np.array([_eval(e) for e in exp_block["lse"]])
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------
# pure-Python brute force (no numpy), written from the definition
# ----------------------------------------------------------------------------

def _brute(q, k, v, block, tau, correction, scale, topk=None):
    N, D = len(q), len(q[0])
    s = scale if scale else 1.0 / math.sqrt(D)
    blocks = []
    start = 0
    while start < N:
        blocks.append((start, min(start + block, N)))
        start += block

    def mean(rows):
        n = len(rows)
        return [sum(r[d] for r in rows) / n for d in range(len(rows[0]))]

    def dot(a, b):
        return sum(x * y for x, y in zip(a, b))

    qbar = [mean(q[a:b]) for a, b in blocks]
    kbar = [mean(k[a:b]) for a, b in blocks]
    vbar = [mean(v[a:b]) for a, b in blocks]
    o = [None] * N
    lse = [None] * N
    for I, (a, b) in enumerate(blocks):
        p = [s * dot(qbar[I], kbar[J]) for J in range(len(blocks))]
        if topk:
            # the topk largest proxies; equal proxies in increasing block order
            ranked = sorted(range(len(blocks)), key=lambda J: (-p[J], J))
            chosen = set(ranked[:topk])
            keep = [J in chosen for J in range(len(blocks))]
        else:
            m = max(p)
            keep = [pj >= m - tau for pj in p]
        for i in range(a, b):
            terms = []  # (logit, multiplicity, value row)
            for J, (c0, c1) in enumerate(blocks):
                if keep[J]:
                    for j in range(c0, c1):
                        terms.append((s * dot(q[i], k[j]), 1.0, v[j]))
                elif correction:
                    terms.append((s * dot(q[i], kbar[J]), float(c1 - c0), vbar[J]))
            M = max(t[0] for t in terms)
            Z = sum(w * math.exp(lg - M) for lg, w, _ in terms)
            o[i] = [sum(w * math.exp(lg - M) * val[d] for lg, w, val in terms) / Z
                    for d in range(len(v[0]))]
            lse[i] = M + math.log(Z)
    return o, lse


@pytest.mark.parametrize("N,block,D", [(7, 2, 1), (12, 4, 3), (16, 4, 5), (13, 4, 2), (9, 3, 4)])
@pytest.mark.parametrize("tau", [0.0, 0.5, 2.0, math.inf])
@pytest.mark.parametrize("corr", [True, False])
def test_brute_force_tiny(N, block, D, tau, corr):
    rng = np.random.default_rng(1000 * N + 10 * D + block)
    q = rng.normal(size=(N, D)) * 1.5
    k = rng.normal(size=(N, D)) * 1.5
    v = rng.normal(size=(N, D + 1))           # Dv != D also allowed by the definition
    o, lse, _ = orc.forward_head(q, k, v, block, tau, corr)
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), block, tau, corr, None)
    np.testing.assert_allclose(o, np.array(ob), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# library special cases (torch float64 on the CPU)
# ----------------------------------------------------------------------------

def _sdpa(q, k, v, bias=None):
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    mask = None if bias is None else torch.from_numpy(bias)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    scores = (qt @ kt.transpose(-1, -2)) / math.sqrt(q.shape[1])
    if mask is not None:
        scores = scores + mask
    return o[0, 0].numpy(), torch.logsumexp(scores, dim=-1)[0, 0].numpy()


def _rand_qkv(seed, N=200, D=16, s=2.0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(N, D)) * s, rng.normal(size=(N, D)) * s, rng.normal(size=(N, D))


@pytest.mark.parametrize("corr", [True, False])
def test_keep_all_equals_sdpa(corr):
    q, k, v = _rand_qkv(1)
    o, lse, keep = orc.forward_head(q, k, v, 64, math.inf, corr)
    assert keep.all()
    o_ref, lse_ref = _sdpa(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


def test_dense_head_equals_sdpa():
    q, k, v = _rand_qkv(2)
    o, lse = orc.dense_head(q, k, v)
    o_ref, lse_ref = _sdpa(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)
    rows = np.array([0, 63, 64, 199])
    o2, lse2 = orc.dense_head(q, k, v, rows=rows)
    np.testing.assert_allclose(o2, o_ref[rows], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tau", [0.0, 1.0, 3.0])
@pytest.mark.parametrize("N", [200, 256, 70])
def test_block_constant_kv_is_exact(tau, N):
    """With block-constant K and V the n_J-copies model is exact: any tau, correction
    on, equals dense softmax attention (ragged tails included: 200 = 3*64 + 8)."""
    rng = np.random.default_rng(3 + N)
    D, block = 16, 64
    Nb = (N + block - 1) // block
    kb = rng.normal(size=(Nb, D)) * 2
    vb = rng.normal(size=(Nb, D))
    k = np.repeat(kb, block, axis=0)[:N]
    v = np.repeat(vb, block, axis=0)[:N]
    q = rng.normal(size=(N, D)) * 2
    o, lse, keep = orc.forward_head(q, k, v, block, tau, True)
    if tau == 0.0 and N > 64:
        assert not keep.all(), "case must skip some blocks to be a pin"
    o_ref, lse_ref = _sdpa(q, k, v)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tau", [0.0, 0.7, 2.5])
@pytest.mark.parametrize("corr", [True, False])
def test_augmented_key_sdpa(tau, corr):
    """The whole method as SDPA over K' = [K; Kbar], V' = [V; Vbar] with an additive bias:
    0 on real keys of kept blocks, ln n_J on the virtual key of a skipped block (if the
    correction is on), -inf elsewhere."""
    q, k, v = _rand_qkv(4 + int(10 * tau), N=300, D=8, s=1.5)
    block = 64
    N = q.shape[0]
    ranges = [(a, min(a + block, N)) for a in range(0, N, block)]
    Nb = len(ranges)
    kbar = np.stack([k[a:b].mean(0) for a, b in ranges])
    vbar = np.stack([v[a:b].mean(0) for a, b in ranges])
    keep, _, _ = orc.route(q, k, block, tau)
    bias = np.full((N, N + Nb), -np.inf)
    for I, (a, b) in enumerate(ranges):
        for J, (c0, c1) in enumerate(ranges):
            if keep[I, J]:
                bias[a:b, c0:c1] = 0.0
            elif corr:
                bias[a:b, N + J] = math.log(c1 - c0)
    o_ref, lse_ref = _sdpa(q, np.concatenate([k, kbar]), np.concatenate([v, vbar]), bias)
    o, lse, _ = orc.forward_head(q, k, v, block, tau, corr)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("tau", [0.0, 1.0, 4.0])
def test_effective_weights_sum_to_one(tau):
    """V = I_N exposes the effective weight of every real key (a skipped block's
    n_J * w spread as w on each of its columns); each row sums to 1.  Shifting V by
    a constant shifts O by the same constant."""
    q, k, _ = _rand_qkv(5, N=150, D=8, s=2.0)
    N = q.shape[0]
    o, _, keep = orc.forward_head(q, k, np.eye(N), 64, tau, True)
    assert (o >= 0).all()
    np.testing.assert_allclose(o.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    rng = np.random.default_rng(6)
    v = rng.normal(size=(N, 8))
    o1, _, _ = orc.forward_head(q, k, v, 64, tau, True)
    o2, _, _ = orc.forward_head(q, k, v + 3.25, 64, tau, True)
    np.testing.assert_allclose(o2, o1 + 3.25, rtol=0, atol=1e-12)


@pytest.mark.parametrize("corr", [True, False])
def test_identical_v_rows(corr):
    q, k, _ = _rand_qkv(7, N=190, D=8, s=2.0)
    row = np.linspace(-1, 1, 8)
    v = np.tile(row, (190, 1))
    o, _, _ = orc.forward_head(q, k, v, 64, 1.0, corr)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)


def test_permutation_within_blocks():
    q, k, v = _rand_qkv(8, N=256, D=8, s=2.0)
    u = np.ones(8) / math.sqrt(8)
    q = q + 2.0 * u                 # every query block leans along u ...
    k[128:192] -= 3.0 * u           # ... and key block 2 points away from it
    block, tau = 64, 0.5
    keep, _, _ = orc.route(q, k, block, tau)
    o0, lse0, _ = orc.forward_head(q, k, v, block, tau, True)
    rng = np.random.default_rng(9)
    # joint permutation of K/V rows inside every key block
    perm = np.concatenate([a + rng.permutation(64) for a in range(0, 256, 64)])
    o1, lse1, _ = orc.forward_head(q, k[perm], v[perm], block, tau, True)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0, rtol=0, atol=1e-12)
    # independent permutations of K rows and V rows inside a block that every query
    # block skips: only its means enter, so nothing changes
    skipped_by_all = [J for J in range(4) if not keep[:, J].any()]
    assert skipped_by_all, "test data must have a block skipped by every query block"
    J = skipped_by_all[0]
    pk = np.arange(256)
    pv = np.arange(256)
    pk[64 * J:64 * J + 64] = 64 * J + rng.permutation(64)
    pv[64 * J:64 * J + 64] = 64 * J + rng.permutation(64)
    o2, lse2, _ = orc.forward_head(q, k[pk], v[pv], block, tau, True)
    np.testing.assert_allclose(o2, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse0, rtol=0, atol=1e-12)
    # sensitivity: the same independent permutation inside a kept block changes O
    Jk = int(np.argmax(keep.sum(axis=0)))
    pk = np.arange(256)
    pk[64 * Jk:64 * Jk + 64] = 64 * Jk + rng.permutation(64)
    o3, _, _ = orc.forward_head(q, k[pk], v, block, tau, True)
    assert np.abs(o3 - o0).max() > 1e-6


def test_tau_nesting_and_argmax():
    q, k, _ = _rand_qkv(10, N=640, D=8, s=2.0)
    prev = None
    for tau in [0.0, 0.25, 1.0, 2.0, 8.0, math.inf]:
        keep, p, m = orc.route(q, k, 64, tau)
        assert keep.sum(axis=1).min() >= 1
        if tau == 0.0:
            np.testing.assert_array_equal(keep, p == m[:, None])
        if prev is not None:
            assert (prev <= keep).all()
        prev = keep
    assert prev.all()


def test_proxy_is_mean_of_score_block():
    """Bilinearity: s * qbar_I . kbar_J is the mean of the scaled score block S_IJ."""
    q, k, _ = _rand_qkv(11, N=200, D=8, s=2.0)
    p = orc.proxy_scores(q, k, 64)
    S = (q @ k.T) / math.sqrt(8)
    ranges = orc.block_ranges(200, 64)
    for I, (a, b) in enumerate(ranges):
        for J, (c, d) in enumerate(ranges):
            assert abs(p[I, J] - S[a:b, c:d].mean()) < 1e-12


@pytest.mark.parametrize("tau", [0.0, 1.0, 3.0])
def test_jensen_lse_order(tau):
    """n_J e^{mean logit} <= sum of e^{logit} (Jensen), so per row
    lse(correction off) <= lse(correction on) <= lse(dense)."""
    q, k, v = _rand_qkv(12, N=300, D=8, s=2.0)
    _, l_off, _ = orc.forward_head(q, k, v, 64, tau, False)
    _, l_on, _ = orc.forward_head(q, k, v, 64, tau, True)
    _, l_dense = orc.dense_head(q, k, v)
    assert (l_off <= l_on + 1e-12).all()
    assert (l_on <= l_dense + 1e-12).all()


def test_explicit_scale_equals_prescaled_q():
    q, k, v = _rand_qkv(13, N=150, D=8, s=1.0)
    s = 0.9
    o1, l1, k1 = orc.forward_head(q, k, v, 64, 1.0, True, scale=s)
    o2, l2, k2 = orc.forward_head(q * s * math.sqrt(8), k, v, 64, 1.0, True)
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tau", [-1.0, float("nan")])
def test_invalid_tau_rejected(tau):
    q, k, _ = _rand_qkv(14, N=64, D=4)
    with pytest.raises(ValueError):
        orc.route(q, k, 64, tau)


def test_batched_forward_matches_heads():
    rng = np.random.default_rng(15)
    q = rng.normal(size=(2, 2, 130, 8)) * 2
    k = rng.normal(size=(2, 2, 130, 8)) * 2
    v = rng.normal(size=(2, 2, 130, 8))
    o, lse, keep = orc.forward(q, k, v, 64, 1.0, True)
    for b in range(2):
        for h in range(2):
            oh, lh, kh = orc.forward_head(q[b, h], k[b, h], v[b, h], 64, 1.0, True)
            np.testing.assert_array_equal(o[b, h], oh)
            np.testing.assert_array_equal(lse[b, h], lh)
            np.testing.assert_array_equal(keep[b, h], kh)
