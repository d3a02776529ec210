"""The C ABI library loads, exports every declared entry point, and validates
arguments on the host (CPU only: no call here reaches a HIP API, since every
case fails validation, is empty, or only sizes a workspace)."""
import ctypes
import math
import os
import re

import pytest

from block_sparse_attention_route_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa_route.h")

FAKE = 1 << 20   # stands in for an aligned device pointer; never dereferenced on failure paths


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return api.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sa_route.h but not exported"


def test_abi_version(lib):
    assert api.sa_abi_version() == 4


def test_status_strings(lib):
    for code, name in enumerate(api.STATUS):
        assert lib.sa_status_string(code).decode().startswith(name)


def _shape(B=1, H=2, T=2, Hg=8, Wg=9, D=128, N=None):
    N = T * Hg * Wg if N is None else N
    return api.Shape(B, H, N, D, T, Hg, Wg)


def _inputs(qk=api.SA_BF16, v=api.SA_BF16, q=FAKE, k=FAKE, vv=FAKE, qs=None, ks=None):
    return api.Inputs(q, k, vv, qs, ks, qk, v)


def _params(block=64, tau=2.0, corr=1, scale=0.0, topk=0, tile=(0, 0, 0)):
    return api.Params(block, tau, corr, scale, topk, *tile)


def _fwd(lib, sh, pr, inp, o=FAKE, lse=FAKE, kept=None, ws=FAKE, ws_bytes=1 << 40):
    return lib.sa_forward(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(inp), o, lse, kept, ws, ws_bytes, None)


def test_workspace_bytes_layout(lib):
    sh = _shape(B=1, H=3, T=1, Hg=10, Wg=13, D=128)     # N = 130 -> Nb = 3, Nbp = 64
    n = lib.sa_workspace_bytes(ctypes.byref(sh), None, ctypes.byref(_inputs()))
    BH, Nb, Nbp, D = 3, 3, 64, 128

    def a256(x):
        return (x + 255) // 256 * 256
    # means, bf16 key means (two halves) and value means, V regrouped, 256 bytes of group counters
    expect = (3 * a256(BH * Nb * D * 4) + a256(2 * BH * Nbp * D * 2) + a256(BH * Nbp * D * 2)
              + a256(BH * Nb * D * 64 * 2) + 256)
    assert n == expect
    # fp32 path keeps only the fp32 means (and the counters)
    n32 = lib.sa_workspace_bytes(ctypes.byref(sh), None, ctypes.byref(_inputs(api.SA_F32, api.SA_F32)))
    assert n32 == 3 * a256(BH * Nb * D * 4) + 256
    nd = lib.sa_dense_workspace_bytes(ctypes.byref(sh), ctypes.byref(_inputs()))
    assert nd == a256(BH * Nb * D * 64 * 2)
    nd32 = lib.sa_dense_workspace_bytes(ctypes.byref(sh), ctypes.byref(_inputs(api.SA_F32, api.SA_F32)))
    assert nd32 == 0


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), "SA_ERR_SHAPE"),
    (dict(N=100), "SA_ERR_SHAPE"),               # N != T*Hg*Wg
    (dict(T=65, Hg=64, Wg=64), "SA_ERR_SHAPE"),  # N > SA_MAX_N
    (dict(B=-1), "SA_ERR_SHAPE"),
    (dict(B=1, H=1 << 24, T=2, Hg=64, Wg=64), "SA_ERR_SHAPE"),   # B*H*Nb = 2^31 workgroups
])
def test_bad_shapes(lib, kw, code):
    sh = _shape(**kw)
    assert api.status_name(_fwd(lib, sh, _params(), _inputs())) == code
    assert lib.sa_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(block=32), "SA_ERR_PARAM"),
    (dict(tau=-1.0), "SA_ERR_PARAM"),
    (dict(tau=math.nan), "SA_ERR_PARAM"),
    (dict(corr=3), "SA_ERR_PARAM"),
    (dict(corr=-1), "SA_ERR_PARAM"),
    (dict(scale=math.inf), "SA_ERR_PARAM"),
    (dict(topk=-1), "SA_ERR_PARAM"),
    (dict(topk=-5, tau=math.nan), "SA_ERR_PARAM"),
    (dict(tile=(4, 4, 2)), "SA_ERR_PARAM"),        # volume 32
    (dict(tile=(0, 8, 8)), "SA_ERR_PARAM"),        # partly zero
    (dict(tile=(-1, -8, 8)), "SA_ERR_PARAM"),
])
def test_bad_params(lib, kw, code):
    assert api.status_name(_fwd(lib, _shape(), _params(**kw), _inputs())) == code


@pytest.mark.parametrize("kw,code", [
    (dict(qk=api.SA_BF16, v=api.SA_F32), "SA_ERR_DTYPE"),
    (dict(qk=api.SA_F32, v=api.SA_BF16), "SA_ERR_DTYPE"),
    (dict(qk=api.SA_FP8_E4M3, v=api.SA_F32), "SA_ERR_DTYPE"),
    (dict(qk=7, v=api.SA_BF16), "SA_ERR_DTYPE"),
    (dict(qk=api.SA_FP8_E4M3, v=api.SA_BF16), "SA_ERR_DTYPE"),            # fp8 without scales
    (dict(qk=api.SA_BF16, v=api.SA_BF16, qs=FAKE, ks=FAKE), "SA_ERR_DTYPE"),  # scales for bf16
    (dict(q=None), "SA_ERR_NULL"),
    (dict(vv=None), "SA_ERR_NULL"),
    (dict(k=FAKE + 8), "SA_ERR_ALIGN"),
])
def test_bad_inputs(lib, kw, code):
    assert api.status_name(_fwd(lib, _shape(), _params(), _inputs(**kw))) == code


def test_bad_outputs_and_workspace(lib):
    sh, pr, inp = _shape(), _params(), _inputs()
    assert api.status_name(_fwd(lib, sh, pr, inp, o=None)) == "SA_ERR_NULL"
    assert api.status_name(_fwd(lib, sh, pr, inp, lse=None)) == "SA_ERR_NULL"
    assert api.status_name(_fwd(lib, sh, pr, inp, o=FAKE + 4)) == "SA_ERR_ALIGN"
    assert api.status_name(_fwd(lib, sh, pr, inp, kept=FAKE + 2)) == "SA_ERR_ALIGN"
    need = lib.sa_workspace_bytes(ctypes.byref(sh), None, ctypes.byref(inp))
    assert api.status_name(_fwd(lib, sh, pr, inp, ws_bytes=need - 1)) == "SA_ERR_WORKSPACE"
    assert api.status_name(_fwd(lib, sh, pr, inp, ws=None)) == "SA_ERR_NULL"
    assert api.status_name(_fwd(lib, sh, pr, inp, ws=FAKE + 8)) == "SA_ERR_ALIGN"
    # params pointer required by the compute entry points
    st = lib.sa_forward(ctypes.byref(sh), None, ctypes.byref(inp), FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert api.status_name(st) == "SA_ERR_NULL"


def test_route_and_dense_validation(lib):
    sh, pr, inp = _shape(), _params(), _inputs()
    st = lib.sa_route(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(inp), None, None, FAKE, 1 << 40, None)
    assert api.status_name(st) == "SA_ERR_NULL"
    st = lib.sa_dense_forward(ctypes.byref(sh), math.nan, ctypes.byref(inp), FAKE, FAKE, FAKE, 1 << 40, None)
    assert api.status_name(st) == "SA_ERR_PARAM"
    st = lib.sa_dense_forward(ctypes.byref(_shape(D=32)), 0.0, ctypes.byref(inp), FAKE, FAKE, FAKE, 1 << 40, None)
    assert api.status_name(st) == "SA_ERR_SHAPE"
    st = lib.sa_pool(ctypes.byref(sh), ctypes.byref(_params(tau=-2.0)), ctypes.byref(inp), FAKE, 1 << 40, None)
    assert api.status_name(st) == "SA_ERR_PARAM"


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(T=0)])
def test_empty_calls_are_ok_without_pointers(lib, kw):
    sh = _shape(**kw)
    inp = _inputs(q=None, k=None, vv=None)
    assert _fwd(lib, sh, _params(), inp, o=None, lse=None, ws=None, ws_bytes=0) == 0
    st = lib.sa_route(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(inp), None, None, None, 0, None)
    assert st == 0
    st = lib.sa_dense_forward(ctypes.byref(sh), 0.0, ctypes.byref(inp), None, None, None, 0, None)
    assert st == 0
    # the first-order correction: nothing to pool or correct either
    assert _fwd(lib, sh, _params(corr=2), inp, o=None, lse=None, ws=None, ws_bytes=0) == 0
    assert lib.sa_pool(ctypes.byref(sh), ctypes.byref(_params(corr=2)), ctypes.byref(inp), None, 0, None) == 0


def test_params_struct_layout():
    # sa_params in include/sa_route.h: block, tau, correction, scale, topk, tile_t/h/w
    assert ctypes.sizeof(api.Params) == 32
    assert [f[0] for f in api.Params._fields_] == ["block", "tau", "correction", "scale", "topk",
                                                    "tile_t", "tile_h", "tile_w"]


def test_tile_order_with_fp8_is_unsupported(lib):
    inp = _inputs(qk=api.SA_FP8_E4M3, v=api.SA_BF16, qs=FAKE, ks=FAKE)
    st = _fwd(lib, _shape(), _params(tile=(4, 4, 4)), inp)
    assert api.status_name(st) == "SA_ERR_UNSUPPORTED"


def test_first_order_workspace_with_fp8_keys(lib):
    # fp8 Q/K with bf16 V: bf16 values per (query block, key block), as for bf16
    sh = _shape(B=1, H=2, T=1, Hg=10, Wg=13, D=64)       # N = 130: Nb = 3, Nbp = 64
    inp = _inputs(qk=api.SA_FP8_E4M3, v=api.SA_BF16)
    n1 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(inp))
    n2 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(corr=2)), ctypes.byref(inp))
    assert n1 > 0 and n2 - n1 == (2 * 3 * 64 * 64 * 2 + 255) // 256 * 256


def test_first_order_workspace_holds_values_per_block_pair(lib):
    sh = _shape(B=2, H=3, T=1, Hg=10, Wg=13, D=128)     # N = 130: Nb = 3, Nbp = 64
    n1 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(_inputs()))
    n2 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(corr=2)), ctypes.byref(_inputs()))
    assert n2 - n1 == (6 * 3 * 64 * 128 * 2 + 255) // 256 * 256
    # with the 3-D tile order both copies are there
    n3 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(corr=2, tile=(1, 8, 8))),
                                ctypes.byref(_inputs()))
    assert n3 - n2 == (6 * 130 * 128 * 2 + 255) // 256 * 256
    # fp32: float values, [BH][Nb][Nb][D]
    f32 = _inputs(api.SA_F32, api.SA_F32)
    m1 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(f32))
    m2 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(corr=2)), ctypes.byref(f32))
    assert m2 - m1 == (6 * 3 * 3 * 128 * 4 + 255) // 256 * 256


def test_tiled_workspace_holds_k_in_tile_order(lib):
    sh = _shape(B=1, H=3, T=1, Hg=10, Wg=13, D=128)     # N = 130
    n0 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(_inputs()))
    n1 = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(tile=(1, 8, 8))), ctypes.byref(_inputs()))
    assert n1 - n0 == (3 * 130 * 128 * 2 + 255) // 256 * 256
    # fp32 reads K through the order directly: no copy
    f32 = _inputs(api.SA_F32, api.SA_F32)
    assert lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(tile=(1, 8, 8))), ctypes.byref(f32)) == \
        lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(f32))


@pytest.mark.parametrize("sparsity,N,expect", [
    (0.9, 75600, 119),      # Nb = 1182: ceil(118.2)
    (0.9, 640, 1),          # Nb = 10: exactly one block
    (0.75, 512, 2),         # Nb = 8: exactly 2, no rounding up past it
    (0.0, 1000, 16),        # keep every block
    (0.99, 64, 1),          # at least one block
])
def test_budget_blocks(sparsity, N, expect):
    assert api.budget_blocks(sparsity, N) == expect


@pytest.mark.parametrize("sparsity", [-0.1, 1.0, 1.5])
def test_budget_blocks_rejects_out_of_range(sparsity):
    with pytest.raises(ValueError):
        api.budget_blocks(sparsity, 640)


def test_budget_blocks_c_abi(lib):
    assert lib.sa_budget_blocks(75600, 0.8) == 237      # ceil(236.4)
    assert lib.sa_budget_blocks(6400, 0.9) == 10        # (1 - 0.9) * 100 is 10 up to rounding
    assert lib.sa_budget_blocks(0, 0.5) == 0
    assert api.status_name(lib.sa_last_status()) == "SA_ERR_PARAM"
    assert lib.sa_budget_blocks(64, math.nan) == 0


def test_first_order_slab_bounds_the_workspace(lib):
    # per head: Nb * Nbp * D bf16 values; the fewest equal slabs of at most
    # floor(8 GiB / that) heads each (at least one head per slab)
    def slab(H, N, D, dt=api.SA_BF16):
        sh = _shape(B=1, H=H, T=1, Hg=1, Wg=N, D=D)
        return lib.sa_first_order_slab_heads(ctypes.byref(sh), ctypes.byref(_inputs(dt, dt)))
    assert slab(40, 75600, 128) == 20          # 368 MB per head: 23 fit, 2 slabs of 20
    assert slab(32, 171360, 128) == 4          # 1.84 GB per head: 4 fit, 8 slabs of 4
    assert slab(3, 262144, 128) == 2           # exactly 4 GiB per head: 2 fit
    assert slab(5, 262144, 128) == 2           # 3 slabs: 2, 2, 1
    assert slab(2, 1024, 64) == 2              # everything fits
    assert slab(2, 1024, 64, api.SA_F32) == 2
    sh = _shape(B=1, H=40, T=1, Hg=1, Wg=75600, D=128)
    base = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(corr=1)), ctypes.byref(_inputs()))
    fo = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(corr=2)), ctypes.byref(_inputs()))
    assert fo - base == 20 * 1182 * 1216 * 128 * 2


def test_noalloc_rejects_a_workspace_above_its_scratch(lib):
    # 720p: the workspace (about 0.85 GB) exceeds the 256 MiB static scratch;
    # refused on the host, before any HIP call
    sh = _shape(B=1, H=40, T=21, Hg=45, Wg=80, D=128)
    st = lib.sa_forward_noalloc(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(_inputs()),
                                FAKE, FAKE, None, None)
    assert api.status_name(st) == "SA_ERR_WORKSPACE"
    assert b"SA_NOALLOC_SCRATCH_BYTES" in lib.sa_last_error()
    n = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(_inputs()))
    assert n > 256 << 20


def test_last_status_explains_a_zero_size(lib):
    sh = _shape()
    inp = _inputs(qk=api.SA_FP8_E4M3, v=api.SA_BF16)
    n = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params(tile=(4, 4, 4))), ctypes.byref(inp))
    assert n == 0 and api.status_name(lib.sa_last_status()) == "SA_ERR_UNSUPPORTED"
    n = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(_params()), ctypes.byref(_inputs()))
    assert n > 0 and lib.sa_last_status() == 0
    bad = _shape(D=96)
    assert lib.sa_dense_workspace_bytes(ctypes.byref(bad), ctypes.byref(_inputs())) == 0
    assert api.status_name(lib.sa_last_status()) == "SA_ERR_SHAPE"


def _pro(lib, eps=1e-6, base=1e4, inp=None, gq=FAKE, gk=FAKE, qo=FAKE, ko=FAKE):
    sh, pr = _shape(), _params()
    inp = _inputs() if inp is None else inp
    p = api.Prologue(eps, base)
    return lib.sa_qk_prologue(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(p), ctypes.byref(inp),
                              gq, gk, qo, ko, FAKE, 1 << 40, None)


@pytest.mark.parametrize("kw,code", [
    (dict(eps=0.0), "SA_ERR_PARAM"),
    (dict(eps=math.nan), "SA_ERR_PARAM"),
    (dict(base=-1.0), "SA_ERR_PARAM"),
    (dict(base=math.inf), "SA_ERR_PARAM"),
    (dict(gq=None), "SA_ERR_NULL"),
    (dict(ko=None), "SA_ERR_NULL"),
    (dict(qo=FAKE + 4), "SA_ERR_ALIGN"),
    (dict(gk=FAKE + 2), "SA_ERR_ALIGN"),
])
def test_prologue_validation(lib, kw, code):
    assert api.status_name(_pro(lib, **kw)) == code


def test_prologue_needs_bf16(lib):
    st = _pro(lib, inp=_inputs(api.SA_F32, api.SA_F32))
    assert api.status_name(st) == "SA_ERR_UNSUPPORTED"
