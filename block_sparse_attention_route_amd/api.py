"""Python binding of libsa_route (include/sa_route.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels.  This module only
turns torch tensors into device pointers and the current HIP stream, allocates
outputs and workspaces with torch when the caller passes none, and raises on
a nonzero status.  There is no fallback: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "SaError", "load_library", "library_path", "Shape", "Params", "Inputs",
    "sa_abi_version", "sa_workspace_bytes", "sa_dense_workspace_bytes", "sa_pool", "sa_route",
    "sa_forward", "sa_forward_noalloc", "sa_forward_pooled", "sa_dense_forward", "sa_qk_prologue", "status_name",
    "Prologue", "make_params", "budget_blocks", "first_order_slab",
    "SA_F32", "SA_BF16", "SA_FP8_E4M3", "BLOCK", "MAX_NB", "MAX_N",
]

SA_F32, SA_BF16, SA_FP8_E4M3 = 0, 1, 2
BLOCK = 64
MAX_NB = 4096
MAX_N = BLOCK * MAX_NB
STATUS = ["SA_OK", "SA_ERR_NULL", "SA_ERR_SHAPE", "SA_ERR_PARAM", "SA_ERR_DTYPE", "SA_ERR_ALIGN",
          "SA_ERR_WORKSPACE", "SA_ERR_UNSUPPORTED", "SA_ERR_HIP"]

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("SA_ROUTE_LIB", os.path.join(_HERE, "_lib", "libsa_route.so"))


class SaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{status_name(status)}: {detail}")


def status_name(status: int) -> str:
    return STATUS[status] if 0 <= status < len(STATUS) else f"status {status}"


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "N", "D", "T", "Hg", "Wg")]


class Params(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("tau", ctypes.c_float),
                ("correction", ctypes.c_int32), ("scale", ctypes.c_float),
                ("topk", ctypes.c_int32),
                ("tile_t", ctypes.c_int32), ("tile_h", ctypes.c_int32), ("tile_w", ctypes.c_int32)]


class Prologue(ctypes.Structure):
    _fields_ = [("norm_eps", ctypes.c_float), ("rope_base", ctypes.c_float)]


class Inputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("q_scale", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("qk_dtype", ctypes.c_int32), ("v_dtype", ctypes.c_int32)]


_lib = None


def load_library():
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libsa_route.so not found at {path}; build it with "
                           "`python -m block_sparse_attention_route_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, I = ctypes.POINTER(Shape), ctypes.POINTER(Params), ctypes.POINTER(Inputs)
    vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.sa_abi_version.restype = ctypes.c_int32
    lib.sa_abi_version.argtypes = []
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_status_string.argtypes = [st]
    lib.sa_last_error.restype = ctypes.c_char_p
    lib.sa_last_error.argtypes = []
    lib.sa_last_status.restype = st
    lib.sa_last_status.argtypes = []
    lib.sa_workspace_bytes.restype = sz
    lib.sa_workspace_bytes.argtypes = [P, S, I]
    lib.sa_dense_workspace_bytes.restype = sz
    lib.sa_dense_workspace_bytes.argtypes = [P, I]
    lib.sa_first_order_slab_heads.restype = ctypes.c_int64
    lib.sa_first_order_slab_heads.argtypes = [P, I]
    lib.sa_budget_blocks.restype = ctypes.c_int32
    lib.sa_budget_blocks.argtypes = [ctypes.c_int32, ctypes.c_double]
    lib.sa_pool.restype = st
    lib.sa_pool.argtypes = [P, S, I, vp, sz, vp]
    lib.sa_route.restype = st
    lib.sa_route.argtypes = [P, S, I, vp, vp, vp, sz, vp]
    for fn in (lib.sa_forward, lib.sa_forward_pooled):
        fn.restype = st
        fn.argtypes = [P, S, I, vp, vp, vp, vp, sz, vp]
    lib.sa_forward_noalloc.restype = st
    lib.sa_forward_noalloc.argtypes = [P, S, I, vp, vp, vp, vp]
    lib.sa_qk_prologue.restype = st
    lib.sa_qk_prologue.argtypes = [P, S, ctypes.POINTER(Prologue), I, vp, vp, vp, vp, vp, sz, vp]
    lib.sa_dense_forward.restype = st
    lib.sa_dense_forward.argtypes = [P, ctypes.c_float, I, vp, vp, vp, sz, vp]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise SaError(status, load_library().sa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return SA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def make_shape(q: torch.Tensor, grid) -> Shape:
    B, H, N, D = q.shape
    T, Hg, Wg = grid
    return Shape(B, H, N, D, T, Hg, Wg)


def make_params(tau: float, correction=True, scale: float = 0.0, topk: int = 0,
                tile=None) -> Params:
    """correction: False / 0 none, True / 1 the mean copies, 2 the first-order
    correction (every dtype pair)."""
    tt, th, tw = (0, 0, 0) if tile is None else (int(x) for x in tile)
    return Params(BLOCK, float(tau), int(correction), float(scale), int(topk), tt, th, tw)


def budget_blocks(sparsity: float, N: int) -> int:
    """Key blocks kept per query block at a fixed sparsity (fraction of the
    Nb key blocks skipped): ceil((1 - sparsity) * Nb), at least 1 (the
    library's sa_budget_blocks)."""
    lib = load_library()
    n = int(lib.sa_budget_blocks(int(N), float(sparsity)))
    if n == 0:
        raise ValueError(lib.sa_last_error().decode())
    return n


def first_order_slab(q, v) -> int:
    """Heads per slab of the first-order correction (sa_first_order_slab_heads)."""
    lib = load_library()
    B, H, N, D = q.shape
    sh = Shape(B, H, N, D, 1, 1, N)
    inp = Inputs(None, None, None, None, None, _dtype_code(q), _dtype_code(v))
    return int(lib.sa_first_order_slab_heads(ctypes.byref(sh), ctypes.byref(inp)))


def make_inputs(q, k, v, q_scale=None, k_scale=None) -> Inputs:
    return Inputs(_ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _dtype_code(q), _dtype_code(v))


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _nb(N: int) -> int:
    return (N + BLOCK - 1) // BLOCK


def sa_abi_version() -> int:
    return int(load_library().sa_abi_version())


def sa_workspace_bytes(q, k, v, grid, q_scale=None, k_scale=None, tile=None, correction=True) -> int:
    lib = load_library()
    sh = make_shape(q, grid)
    inp = Inputs(None, None, None, None, None, _dtype_code(q), _dtype_code(v))
    pr = make_params(math.inf, correction, 0.0, 0, tile)
    n = lib.sa_workspace_bytes(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(inp))
    if n == 0 and sh.B * sh.H * sh.N > 0:
        raise SaError(int(lib.sa_last_status()), lib.sa_last_error().decode() or "invalid arguments")
    return int(n)


def sa_dense_workspace_bytes(q, k, v, grid) -> int:
    lib = load_library()
    sh = make_shape(q, grid)
    inp = Inputs(None, None, None, None, None, _dtype_code(q), _dtype_code(v))
    return int(lib.sa_dense_workspace_bytes(ctypes.byref(sh), ctypes.byref(inp)))


def _workspace(nbytes: int, like: torch.Tensor, ws: torch.Tensor | None) -> torch.Tensor:
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)
    return ws


def sa_pool(q, k, v, grid, *, tau: float = math.inf, correction=True, scale: float = 0.0,
            workspace: torch.Tensor | None = None, q_scale=None, k_scale=None, topk: int = 0,
            tile=None) -> torch.Tensor:
    """Step pool: block means (and V regrouped per 64-key block) into the
    workspace."""
    lib = load_library()
    ws = _workspace(sa_workspace_bytes(q, k, v, grid, q_scale, k_scale, tile, correction), q, workspace)
    sh, pr, inp = make_shape(q, grid), make_params(tau, correction, scale, topk, tile), make_inputs(q, k, v, q_scale, k_scale)
    _check(lib.sa_pool(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(inp), _ptr(ws), ws.numel(), _stream(q)))
    return ws


def sa_route(q, k, v, grid, *, tau: float = math.inf, scale: float = 0.0, workspace=None, q_scale=None,
             k_scale=None, mask=None, kept=None, topk: int = 0, tile=None):
    """Steps pool + route: returns (mask uint8 [B,H,Nb,Nb], kept int32 [B,H,Nb])."""
    lib = load_library()
    B, H, N, _ = q.shape
    Nb = _nb(N)
    ws = _workspace(sa_workspace_bytes(q, k, v, grid, q_scale, k_scale, tile), q, workspace)
    if mask is None:
        mask = torch.empty((B, H, Nb, Nb), dtype=torch.uint8, device=q.device)
    if kept is None:
        kept = torch.empty((B, H, Nb), dtype=torch.int32, device=q.device)
    sh, pr, inp = make_shape(q, grid), make_params(tau, True, scale, topk, tile), make_inputs(q, k, v, q_scale, k_scale)
    _check(lib.sa_route(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(inp), _ptr(mask), _ptr(kept),
                        _ptr(ws), ws.numel(), _stream(q)))
    return mask, kept


def _outs(q, v, out, lse, want_kept, kept):
    B, H, N, D = q.shape
    if out is None:
        out = torch.empty((B, H, N, D), dtype=v.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if want_kept and kept is None:
        kept = torch.empty((B, H, _nb(N)), dtype=torch.int32, device=q.device)
    return out, lse, kept


def sa_forward(q, k, v, grid, *, tau: float = math.inf, correction=True, scale: float = 0.0,
               workspace=None, q_scale=None, k_scale=None, out=None, lse=None, want_kept=False,
               kept=None, topk: int = 0, tile=None):
    """Pool + fused routed sparse attention with correction: returns (o, lse, kept or None)."""
    lib = load_library()
    ws = _workspace(sa_workspace_bytes(q, k, v, grid, q_scale, k_scale, tile, correction), q, workspace)
    out, lse, kept = _outs(q, v, out, lse, want_kept, kept)
    sh, pr, inp = make_shape(q, grid), make_params(tau, correction, scale, topk, tile), make_inputs(q, k, v, q_scale, k_scale)
    _check(lib.sa_forward(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(inp), _ptr(out), _ptr(lse),
                          _ptr(kept), _ptr(ws), ws.numel(), _stream(q)))
    return out, lse, kept


def sa_forward_noalloc(q, k, v, grid, *, tau: float = math.inf, correction=True, scale: float = 0.0,
                       q_scale=None, k_scale=None, out=None, lse=None, want_kept=False, kept=None,
                       topk: int = 0, tile=None):
    """sa_forward with the library's static scratch as the workspace (no
    device allocation by the library; outputs are allocated here when not
    given).  Returns (o, lse, kept or None)."""
    lib = load_library()
    out, lse, kept = _outs(q, v, out, lse, want_kept, kept)
    sh, pr, inp = make_shape(q, grid), make_params(tau, correction, scale, topk, tile), make_inputs(q, k, v, q_scale, k_scale)
    _check(lib.sa_forward_noalloc(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(inp), _ptr(out), _ptr(lse),
                                  _ptr(kept), _stream(q)))
    return out, lse, kept


def sa_forward_pooled(q, k, v, grid, *, tau: float = math.inf, correction=True, scale: float = 0.0,
                      workspace, q_scale=None, k_scale=None, out=None, lse=None, want_kept=False,
                      kept=None, topk: int = 0, tile=None):
    """The fused kernel alone; `workspace` must hold sa_pool's output for these inputs."""
    lib = load_library()
    out, lse, kept = _outs(q, v, out, lse, want_kept, kept)
    sh, pr, inp = make_shape(q, grid), make_params(tau, correction, scale, topk, tile), make_inputs(q, k, v, q_scale, k_scale)
    _check(lib.sa_forward_pooled(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(inp), _ptr(out), _ptr(lse),
                                 _ptr(kept), _ptr(workspace), workspace.numel(), _stream(q)))
    return out, lse, kept


def sa_qk_prologue(xq, xk, v, grid, q_gain, k_gain, *, norm_eps: float = 1e-6, rope_base: float = 10000.0,
                   tau: float = math.inf, topk: int = 0, tile=None, correction=True, scale: float = 0.0,
                   workspace=None, q_out=None, k_out=None):
    """Fused producer step: RMS norm + gain + 3-D rotary embedding of the raw
    Q/K projections (bf16) into q_out / k_out, with the pool's workspace
    filled from them.  Returns (q_out, k_out, workspace); follow with
    sa_forward_pooled(q_out, k_out, v, ...) using the same tau/topk/tile/correction/scale."""
    lib = load_library()
    ws = _workspace(sa_workspace_bytes(xq, xk, v, grid, tile=tile, correction=correction), xq, workspace)
    if q_out is None:
        q_out = torch.empty_like(xq)
    if k_out is None:
        k_out = torch.empty_like(xk)
    sh, pr, inp = make_shape(xq, grid), make_params(tau, correction, scale, topk, tile), make_inputs(xq, xk, v)
    pro = Prologue(float(norm_eps), float(rope_base))
    _check(lib.sa_qk_prologue(ctypes.byref(sh), ctypes.byref(pr), ctypes.byref(pro), ctypes.byref(inp),
                              _ptr(q_gain), _ptr(k_gain), _ptr(q_out), _ptr(k_out), _ptr(ws), ws.numel(),
                              _stream(xq)))
    return q_out, k_out, ws


def sa_dense_forward(q, k, v, grid, *, scale: float = 0.0, workspace=None, q_scale=None, k_scale=None,
                     out=None, lse=None):
    """Dense softmax attention (the tau = inf limit): returns (o, lse)."""
    lib = load_library()
    n = sa_dense_workspace_bytes(q, k, v, grid)
    ws = _workspace(n, q, workspace) if n else workspace
    out, lse, _ = _outs(q, v, out, lse, False, None)
    sh, inp = make_shape(q, grid), make_inputs(q, k, v, q_scale, k_scale)
    _check(lib.sa_dense_forward(ctypes.byref(sh), float(scale), ctypes.byref(inp), _ptr(out), _ptr(lse),
                                _ptr(ws) if ws is not None else None, ws.numel() if ws is not None else 0,
                                _stream(q)))
    return out, lse
