"""Thin ctypes binding of libssa_mi355x.so (argument marshalling only).

Every function here has the name of the C entry point it calls, checks that
the tensors it is given match the layout the C ABI documents, allocates
outputs and workspace with torch (device memory is torch's plumbing), and
passes raw device pointers and torch's current HIP stream.  All computation
happens in the library's HIP kernels; there is no fallback: if the library is
missing, importing this module's functions raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SSA_MI355X_LIB", os.path.join(HERE, "libssa_mi355x.so"))

SSA_OK, SSA_ERR_INVALID_ARGUMENT, SSA_ERR_UNSUPPORTED, SSA_ERR_WORKSPACE_TOO_SMALL, SSA_ERR_HIP = range(5)
SSA_F32, SSA_BF16 = 0, 1
(SSA_OP_ROUTE, SSA_OP_ATTN, SSA_OP_DECODE, SSA_OP_ROUTE_TILES, SSA_OP_TILE_ATTN,
 SSA_OP_ATTN_BWD, SSA_OP_ROUTE_HIER) = 1, 2, 3, 4, 5, 6, 7

_vp = ctypes.c_void_p


class SSAParams(ctypes.Structure):
    """Mirror of ssa_params (include/ssa.h)."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seq_len", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("beta", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
    ]


class SSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (loads on first use; raises if it was not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m content_routed_block_stats_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(SSAParams)
    L.ssa_block_stats.argtypes = [P, _vp, _vp, _vp, _vp]
    L.ssa_workspace_size.argtypes = [P, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    L.ssa_route_topk.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.ssa_route_tempered.argtypes = [P, _vp, _vp, _vp, _vp, _vp]
    L.ssa_route_tiles.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.ssa_tile_attn_fwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.ssa_sparse_attn_bwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_size_t, _vp]
    L.ssa_sparse_attn_fwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    L.ssa_decode_step.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp]
    L.ssa_decode_step_noalloc.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp]
    L.ssa_group_stats.argtypes = [P, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp]
    L.ssa_route_hier.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                 _vp, ctypes.c_size_t, _vp]
    L.ssa_route_hier_prefill_workspace_size.argtypes = [P, ctypes.c_int32,
                                                        ctypes.POINTER(ctypes.c_size_t)]
    L.ssa_route_hier_prefill.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp,
                                         _vp, _vp, ctypes.c_size_t, _vp]
    L.ssa_probe_mfma_bf16.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_double), _vp]
    L.ssa_probe_hbm_read.argtypes = [_vp, ctypes.c_size_t, _vp, ctypes.c_int32, _vp]
    for name in ("ssa_block_stats", "ssa_workspace_size", "ssa_route_topk", "ssa_route_tempered",
                 "ssa_route_tiles", "ssa_tile_attn_fwd", "ssa_sparse_attn_fwd",
                 "ssa_sparse_attn_bwd", "ssa_decode_step", "ssa_decode_step_noalloc",
                 "ssa_group_stats", "ssa_route_hier", "ssa_route_hier_prefill_workspace_size",
                 "ssa_route_hier_prefill", "ssa_probe_mfma_bf16",
                 "ssa_probe_hbm_read"):
        getattr(L, name).restype = ctypes.c_int
    L.ssa_status_string.argtypes = [ctypes.c_int]
    L.ssa_status_string.restype = ctypes.c_char_p
    L.ssa_last_error.argtypes = []
    L.ssa_last_error.restype = ctypes.c_char_p
    L.ssa_version.argtypes = []
    L.ssa_version.restype = ctypes.c_int32
    _LIB = L
    return L


def status_string(status: int) -> str:
    return lib().ssa_status_string(status).decode()


def _check(status: int) -> None:
    if status != SSA_OK:
        raise SSAError(status, lib().ssa_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return SSA_F32
    if t == torch.bfloat16:
        return SSA_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev_check(*tensors: torch.Tensor) -> None:
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def make_params(*, batch, n_q_heads, n_kv_heads, head_dim, seq_len, block_size, top_k=0,
                window=1, beta=2.0, scale=None, in_dtype=torch.bfloat16,
                out_dtype=None) -> SSAParams:
    if scale is None:
        scale = float(1.0 / math.sqrt(head_dim))
    return SSAParams(batch, n_q_heads, n_kv_heads, head_dim, seq_len, block_size, top_k, window,
                     beta, scale, _dtype_code(in_dtype),
                     _dtype_code(out_dtype if out_dtype is not None else in_dtype))


def ssa_workspace_size(p: SSAParams, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ssa_workspace_size(ctypes.byref(p), op, ctypes.byref(n)))
    return n.value


def _workspace(p: SSAParams, op: int, device, workspace: torch.Tensor | None) -> torch.Tensor:
    need = ssa_workspace_size(p, op)
    if workspace is not None and workspace.numel() >= need:
        return workspace
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


def ssa_block_stats(K: torch.Tensor, block_size: int, *, mu: torch.Tensor | None = None,
                    sigma: torch.Tensor | None = None):
    """K [b, Hkv, n, d] -> (mu [b, Hkv, nb, d], sigma [b, Hkv, nb, d, d]) float32."""
    _dev_check(K)
    b, hkv, n, d = K.shape
    nb = n // block_size
    if mu is None:
        mu = torch.empty((b, hkv, nb, d), dtype=torch.float32, device=K.device)
    if sigma is None:
        sigma = torch.empty((b, hkv, nb, d, d), dtype=torch.float32, device=K.device)
    _dev_check(mu, sigma)
    p = make_params(batch=b, n_q_heads=hkv, n_kv_heads=hkv, head_dim=d, seq_len=n,
                    block_size=block_size, in_dtype=K.dtype)
    _check(lib().ssa_block_stats(ctypes.byref(p), _ptr(K), _ptr(mu), _ptr(sigma), _stream()))
    return mu, sigma


def ssa_route_topk(Q: torch.Tensor, mu: torch.Tensor, sigma: torch.Tensor, *, block_size: int,
                   top_k: int, beta: float = 2.0, want_kth: bool = False,
                   idx: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Q [b, Hq, n, d], stats of [b, Hkv, nb, ...] -> idx [b, Hq, n, k] int32 (, kth [.., 2])."""
    _dev_check(Q, mu, sigma)
    b, hq, n, d = Q.shape
    hkv = mu.shape[1]
    if mu.shape[:2] != (b, hkv) or mu.shape[2] != n // block_size or mu.shape[3] != d:
        raise ValueError("mu does not match Q and block_size")
    if sigma.shape != (*mu.shape, d):
        raise ValueError("sigma does not match mu")
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                    block_size=block_size, top_k=top_k, beta=beta, in_dtype=Q.dtype)
    if idx is None:
        idx = torch.empty((b, hq, n, top_k), dtype=torch.int32, device=Q.device)
    kth = torch.empty((b, hq, n, 2), dtype=torch.float32, device=Q.device) if want_kth else None
    ws = _workspace(p, SSA_OP_ROUTE, Q.device, workspace)
    _check(lib().ssa_route_topk(ctypes.byref(p), _ptr(Q), _ptr(mu), _ptr(sigma), _ptr(idx),
                                _ptr(kth), _ptr(ws), ws.numel(), _stream()))
    return (idx, kth) if want_kth else idx


def ssa_route_tempered(Q: torch.Tensor, K: torch.Tensor, *, block_size: int, top_k: int,
                       beta: float, want_kth: bool = False, idx: torch.Tensor | None = None):
    """Exact tempered routing: Q [b, Hq, n, d], K [b, Hkv, n, d] -> idx [b, Hq, n, k] int32
    (, kth [.., 2]): top-k of (1/beta) ln mean_j exp(beta q.k_j) over routable blocks."""
    _dev_check(Q, K)
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    if K.shape != (b, hkv, n, d) or K.dtype != Q.dtype:
        raise ValueError("K does not match Q")
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                    block_size=block_size, top_k=top_k, beta=beta, in_dtype=Q.dtype)
    if idx is None:
        idx = torch.empty((b, hq, n, top_k), dtype=torch.int32, device=Q.device)
    kth = torch.empty((b, hq, n, 2), dtype=torch.float32, device=Q.device) if want_kth else None
    _check(lib().ssa_route_tempered(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(idx), _ptr(kth),
                                    _stream()))
    return (idx, kth) if want_kth else idx


def ssa_route_tiles(Q: torch.Tensor, mu: torch.Tensor, sigma: torch.Tensor, *, block_size: int,
                    top_k: int, beta: float = 2.0, want_kth: bool = False,
                    idx: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Query-tile-shared routing: Q [b, Hq, n, d], block statistics -> idx
    [b, Hq, ceil(n/B), k] int32 (, kth [.., 2]), one selection per tile of B positions."""
    _dev_check(Q, mu, sigma)
    b, hq, n, d = Q.shape
    hkv = mu.shape[1]
    if mu.shape[:2] != (b, hkv) or mu.shape[2] != n // block_size or mu.shape[3] != d:
        raise ValueError("mu does not match Q and block_size")
    if sigma.shape != (*mu.shape, d):
        raise ValueError("sigma does not match mu")
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                    block_size=block_size, top_k=top_k, beta=beta, in_dtype=Q.dtype)
    tiles = (n + block_size - 1) // block_size
    if idx is None:
        idx = torch.empty((b, hq, tiles, top_k), dtype=torch.int32, device=Q.device)
    kth = torch.empty((b, hq, tiles, 2), dtype=torch.float32, device=Q.device) if want_kth else None
    ws = _workspace(p, SSA_OP_ROUTE_TILES, Q.device, workspace)
    _check(lib().ssa_route_tiles(ctypes.byref(p), _ptr(Q), _ptr(mu), _ptr(sigma), _ptr(idx),
                                 _ptr(kth), _ptr(ws), ws.numel(), _stream()))
    return (idx, kth) if want_kth else idx


def ssa_tile_attn_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor, *,
                      block_size: int, window: int, scale: float | None = None,
                      out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
                      lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Exact softmax over each tile's selected blocks + the row's window -> (O, lse)."""
    _dev_check(Q, K, V, idx)
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    if K.shape != (b, hkv, n, d) or V.shape != K.shape:
        raise ValueError("K/V do not match Q")
    tiles = (n + block_size - 1) // block_size
    if idx.dtype != torch.int32 or idx.shape[:3] != (b, hq, tiles):
        raise ValueError("idx must be int32 [b, Hq, ceil(n/B), k]")
    top_k = idx.shape[3]
    out_dtype = out_dtype or Q.dtype
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                    block_size=block_size, top_k=top_k, window=window, scale=scale,
                    in_dtype=Q.dtype, out_dtype=out_dtype)
    if out is None:
        out = torch.empty((b, hq, n, d), dtype=out_dtype, device=Q.device)
    if lse is None:
        lse = torch.empty((b, hq, n), dtype=torch.float32, device=Q.device)
    ws = _workspace(p, SSA_OP_TILE_ATTN, Q.device, workspace)
    _check(lib().ssa_tile_attn_fwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx),
                                   _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return out, lse


def ssa_sparse_attn_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor, *,
                        block_size: int, window: int, scale: float | None = None,
                        out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Exact softmax over selected blocks + window -> (O [b, Hq, n, d], lse [b, Hq, n] float32)."""
    _dev_check(Q, K, V, idx)
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    if K.shape != (b, hkv, n, d) or V.shape != K.shape:
        raise ValueError("K/V do not match Q")
    if idx.dtype != torch.int32 or idx.shape[:3] != (b, hq, n):
        raise ValueError("idx must be int32 [b, Hq, n, k]")
    top_k = idx.shape[3]
    out_dtype = out_dtype or Q.dtype
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                    block_size=block_size, top_k=top_k, window=window, scale=scale,
                    in_dtype=Q.dtype, out_dtype=out_dtype)
    if out is None:
        out = torch.empty((b, hq, n, d), dtype=out_dtype, device=Q.device)
    if lse is None:
        lse = torch.empty((b, hq, n), dtype=torch.float32, device=Q.device)
    ws = _workspace(p, SSA_OP_ATTN, Q.device, workspace)
    _check(lib().ssa_sparse_attn_fwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx),
                                     _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return out, lse


def ssa_sparse_attn_bwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor,
                        O: torch.Tensor, lse: torch.Tensor, dO: torch.Tensor, *, block_size: int,
                        window: int, scale: float | None = None,
                        workspace: torch.Tensor | None = None):
    """Gradients through the sparse attention with fixed selections:
    (dQ [b, Hq, n, d], dK, dV [b, Hkv, n, d]) float32, given the forward's O and lse
    and the upstream gradient dO (same dtype as Q)."""
    _dev_check(Q, K, V, idx, O, lse, dO)
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    if K.shape != (b, hkv, n, d) or V.shape != K.shape:
        raise ValueError("K/V do not match Q")
    if idx.dtype != torch.int32 or idx.shape[:3] != (b, hq, n):
        raise ValueError("idx must be int32 [b, Hq, n, k]")
    if O.shape != Q.shape or dO.shape != Q.shape or dO.dtype != Q.dtype:
        raise ValueError("O and dO must be [b, Hq, n, d], dO in Q's dtype")
    if lse.shape != (b, hq, n) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [b, Hq, n]")
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                    block_size=block_size, top_k=idx.shape[3], window=window, scale=scale,
                    in_dtype=Q.dtype, out_dtype=O.dtype)
    dQ = torch.empty((b, hq, n, d), dtype=torch.float32, device=Q.device)
    dK = torch.empty((b, hkv, n, d), dtype=torch.float32, device=Q.device)
    dV = torch.empty((b, hkv, n, d), dtype=torch.float32, device=Q.device)
    ws = _workspace(p, SSA_OP_ATTN_BWD, Q.device, workspace)
    _check(lib().ssa_sparse_attn_bwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(idx), _ptr(O),
                                     _ptr(lse), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ws),
                                     ws.numel(), _stream()))
    return dQ, dK, dV


def ssa_decode_step(q, k_new, v_new, K_cache, V_cache, cache_len, mu, sigma, *, block_size: int,
                    top_k: int, window: int, beta: float = 2.0, scale: float | None = None,
                    out_dtype: torch.dtype | None = None, return_idx: bool = False,
                    workspace: torch.Tensor | None = None):
    """One decode step (appends, updates stats on block completion, bumps cache_len).

    q [b, Hq, d]; k_new/v_new [b, Hkv, d]; caches [b, Hkv, C, d]; cache_len [b] int32
    (device); mu [b, Hkv, C/B, d]; sigma [b, Hkv, C/B, d, d].  Returns (o, lse[, idx]).
    """
    _dev_check(q, k_new, v_new, K_cache, V_cache, cache_len, mu, sigma)
    b, hq, d = q.shape
    hkv, cap = K_cache.shape[1], K_cache.shape[2]
    if K_cache.shape != (b, hkv, cap, d) or V_cache.shape != K_cache.shape:
        raise ValueError("caches do not match q")
    if k_new.shape != (b, hkv, d) or v_new.shape != (b, hkv, d):
        raise ValueError("k_new/v_new must be [b, Hkv, d]")
    if cache_len.dtype != torch.int32 or cache_len.shape != (b,):
        raise ValueError("cache_len must be int32 [b]")
    if mu.shape != (b, hkv, cap // block_size, d) or sigma.shape != (*mu.shape, d):
        raise ValueError("stats do not match the cache capacity")
    out_dtype = out_dtype or q.dtype
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=cap,
                    block_size=block_size, top_k=top_k, window=window, beta=beta, scale=scale,
                    in_dtype=q.dtype, out_dtype=out_dtype)
    o = torch.empty((b, hq, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((b, hq), dtype=torch.float32, device=q.device)
    idx = torch.empty((b, hq, top_k), dtype=torch.int32, device=q.device) if return_idx else None
    ws = _workspace(p, SSA_OP_DECODE, q.device, workspace)
    _check(lib().ssa_decode_step(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(K_cache),
                                 _ptr(V_cache), _ptr(cache_len), _ptr(mu), _ptr(sigma), _ptr(idx),
                                 _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return (o, lse, idx) if return_idx else (o, lse)


def ssa_decode_step_noalloc(q, k_new, v_new, K_cache, V_cache, cache_len, mu, sigma, *,
                            block_size: int, top_k: int, window: int, beta: float = 2.0,
                            scale: float | None = None, out_dtype: torch.dtype | None = None,
                            out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                            idx: torch.Tensor | None = None):
    """ssa_decode_step without a workspace: the library's own scratch array is
    used, so the C call allocates nothing.  Outputs (o, lse, idx) may be passed
    in so the Python side allocates nothing either.  Returns (o, lse[, idx])."""
    _dev_check(q, k_new, v_new, K_cache, V_cache, cache_len, mu, sigma, out, lse, idx)
    b, hq, d = q.shape
    hkv, cap = K_cache.shape[1], K_cache.shape[2]
    if K_cache.shape != (b, hkv, cap, d) or V_cache.shape != K_cache.shape:
        raise ValueError("caches do not match q")
    if k_new.shape != (b, hkv, d) or v_new.shape != (b, hkv, d):
        raise ValueError("k_new/v_new must be [b, Hkv, d]")
    if cache_len.dtype != torch.int32 or cache_len.shape != (b,):
        raise ValueError("cache_len must be int32 [b]")
    if mu.shape != (b, hkv, cap // block_size, d) or sigma.shape != (*mu.shape, d):
        raise ValueError("stats do not match the cache capacity")
    out_dtype = out.dtype if out is not None else (out_dtype or q.dtype)
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=cap,
                    block_size=block_size, top_k=top_k, window=window, beta=beta, scale=scale,
                    in_dtype=q.dtype, out_dtype=out_dtype)
    if out is None:
        out = torch.empty((b, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((b, hq), dtype=torch.float32, device=q.device)
    if out.shape != (b, hq, d) or lse.shape != (b, hq) or lse.dtype != torch.float32:
        raise ValueError("out must be [b, Hq, d], lse float32 [b, Hq]")
    if idx is not None and (idx.shape != (b, hq, top_k) or idx.dtype != torch.int32):
        raise ValueError("idx must be int32 [b, Hq, k]")
    _check(lib().ssa_decode_step_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_new), _ptr(v_new),
                                         _ptr(K_cache), _ptr(V_cache), _ptr(cache_len), _ptr(mu),
                                         _ptr(sigma), _ptr(idx), _ptr(out), _ptr(lse), _stream()))
    return (out, lse, idx) if idx is not None else (out, lse)


def ssa_group_stats(mu: torch.Tensor, sigma: torch.Tensor, *, block_size: int, group_blocks: int):
    """Stats mu [b, Hkv, nb, d], sigma [b, Hkv, nb, d, d] -> group summaries
    (gmu [b, Hkv, G, d], gsigma [b, Hkv, G, d, d], grl [b, Hkv, G, 2]) float32,
    G = ceil(nb / group_blocks)."""
    _dev_check(mu, sigma)
    b, hkv, nb, d = mu.shape
    if sigma.shape != (*mu.shape, d) or mu.dtype != torch.float32 or sigma.dtype != torch.float32:
        raise ValueError("mu/sigma must be float32 [b, Hkv, nb, d] / [b, Hkv, nb, d, d]")
    if group_blocks < 1:
        raise ValueError("group_blocks must be positive")
    G = -(-nb // group_blocks)
    gmu = torch.empty((b, hkv, G, d), dtype=torch.float32, device=mu.device)
    gsigma = torch.empty((b, hkv, G, d, d), dtype=torch.float32, device=mu.device)
    grl = torch.empty((b, hkv, G, 2), dtype=torch.float32, device=mu.device)
    if nb == 0:
        return gmu, gsigma, grl
    p = make_params(batch=b, n_q_heads=hkv, n_kv_heads=hkv, head_dim=d, seq_len=nb * block_size,
                    block_size=block_size, in_dtype=torch.float32)
    _check(lib().ssa_group_stats(ctypes.byref(p), _ptr(mu), _ptr(sigma), group_blocks, _ptr(gmu),
                                 _ptr(gsigma), _ptr(grl), _stream()))
    return gmu, gsigma, grl


def ssa_route_hier(q: torch.Tensor, mu: torch.Tensor, sigma: torch.Tensor, gmu: torch.Tensor,
                   gsigma: torch.Tensor, grl: torch.Tensor, pos: torch.Tensor, *, block_size: int,
                   group_blocks: int, top_k: int, beta: float = 2.0, want_evaluated: bool = False,
                   idx: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Exact top-k of decode queries q [b, Hq, d] at positions pos [b] (int32)
    by branch and bound over block groups -> idx [b, Hq, k] int32 (, evaluated
    [b, Hkv] int32).  mu/sigma hold nb block slots; gmu/gsigma/grl come from
    ssa_group_stats with the same group_blocks."""
    _dev_check(q, mu, sigma, gmu, gsigma, grl, pos)
    b, hq, d = q.shape
    hkv, nb = mu.shape[1], mu.shape[2]
    if mu.shape != (b, hkv, nb, d) or sigma.shape != (*mu.shape, d):
        raise ValueError("mu/sigma do not match q")
    if group_blocks < 1:
        raise ValueError("group_blocks must be positive")
    G = -(-nb // group_blocks)
    if gmu.shape != (b, hkv, G, d) or gsigma.shape != (b, hkv, G, d, d) or grl.shape != (b, hkv, G, 2):
        raise ValueError("group summaries do not match mu")
    if pos.dtype != torch.int32 or pos.shape != (b,):
        raise ValueError("pos must be int32 [b]")
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=nb * block_size,
                    block_size=block_size, top_k=top_k, beta=beta, in_dtype=q.dtype)
    if idx is None:
        idx = torch.empty((b, hq, top_k), dtype=torch.int32, device=q.device)
    ev = torch.empty((b, hkv), dtype=torch.int32, device=q.device) if want_evaluated else None
    ws = _workspace(p, SSA_OP_ROUTE_HIER, q.device, workspace)
    _check(lib().ssa_route_hier(ctypes.byref(p), _ptr(q), _ptr(mu), _ptr(sigma), _ptr(gmu),
                                _ptr(gsigma), _ptr(grl), group_blocks, _ptr(pos), _ptr(idx),
                                _ptr(ev), _ptr(ws), ws.numel(), _stream()))
    return (idx, ev) if want_evaluated else idx


def ssa_route_hier_prefill_workspace_size(p: SSAParams, group_blocks: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ssa_route_hier_prefill_workspace_size(ctypes.byref(p), group_blocks,
                                                       ctypes.byref(n)))
    return n.value


def route_tile_count(seq_len: int, n_q_heads: int, n_kv_heads: int) -> int:
    """512-row tiles per (sequence, KV head) of ssa_route_hier_prefill's rows."""
    return -(-seq_len * (n_q_heads // n_kv_heads) // 512)


def ssa_route_hier_prefill(Q: torch.Tensor, mu: torch.Tensor, sigma: torch.Tensor,
                           gmu: torch.Tensor, gsigma: torch.Tensor, grl: torch.Tensor, *,
                           block_size: int, group_blocks: int, top_k: int, beta: float = 2.0,
                           want_evaluated: bool = False, idx: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None):
    """Exact top-k of prefill rows Q [b, Hq, n, d] (bfloat16) by branch and
    bound over groups -> idx [b, Hq, n, k] int32 (, evaluated [b, Hkv, tiles]
    int32: blocks scored per 512-row tile).  gmu/gsigma/grl come from
    ssa_group_stats of mu/sigma with the same group_blocks."""
    _dev_check(Q, mu, sigma, gmu, gsigma, grl)
    b, hq, n, d = Q.shape
    hkv, nb = mu.shape[1], mu.shape[2]
    if mu.shape != (b, hkv, nb, d) or sigma.shape != (*mu.shape, d):
        raise ValueError("mu/sigma do not match Q")
    if nb != n // block_size:
        raise ValueError("mu/sigma must hold n // block_size blocks")
    if group_blocks < 1:
        raise ValueError("group_blocks must be positive")
    G = -(-nb // group_blocks)
    if gmu.shape != (b, hkv, G, d) or gsigma.shape != (b, hkv, G, d, d) or grl.shape != (b, hkv, G, 2):
        raise ValueError("group summaries do not match mu")
    p = make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                    block_size=block_size, top_k=top_k, beta=beta, in_dtype=Q.dtype)
    if idx is None:
        idx = torch.empty((b, hq, n, top_k), dtype=torch.int32, device=Q.device)
    ev = (torch.empty((b, hkv, route_tile_count(n, hq, hkv)), dtype=torch.int32, device=Q.device)
          if want_evaluated else None)
    need = ssa_route_hier_prefill_workspace_size(p, group_blocks)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=Q.device)
    _check(lib().ssa_route_hier_prefill(ctypes.byref(p), _ptr(Q), _ptr(mu), _ptr(sigma), _ptr(gmu),
                                        _ptr(gsigma), _ptr(grl), group_blocks, _ptr(idx), _ptr(ev),
                                        _ptr(workspace), workspace.numel(), _stream()))
    return (idx, ev) if want_evaluated else idx


# -- peak probes (include/ssa_probes.h) ----------------------------------------

def ssa_probe_mfma_bf16(workgroups: int, iters: int, device="cuda"):
    """Launch the dense bf16 MFMA loop on the current stream -> (out, flops)."""
    out = torch.empty((workgroups,), dtype=torch.float32, device=device)
    fl = ctypes.c_double(0.0)
    _check(lib().ssa_probe_mfma_bf16(_ptr(out), workgroups, iters, ctypes.byref(fl), _stream()))
    return out, fl.value


def ssa_probe_hbm_read(buf: torch.Tensor, workgroups: int, out: torch.Tensor | None = None):
    """Launch the streaming read of buf (contiguous, on the GPU) on the current
    stream -> out (uint32 as int32, [workgroups * 256])."""
    _dev_check(buf)
    if out is None:
        out = torch.empty((workgroups * 256,), dtype=torch.int32, device=buf.device)
    _check(lib().ssa_probe_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                                    workgroups, _stream()))
    return out
