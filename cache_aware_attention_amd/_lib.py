"""Thin ctypes binding of libmarca (argument marshalling only).

Every function below has the name of the C entry point it calls.  It checks
that tensors live on the GPU with the dtype and shape the call needs, passes
raw device pointers and the current HIP stream, and turns a negative status
into MarError.  All computation happens in the library's HIP kernels; there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path
from typing import Optional

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libmarca.so"

MAR_OK = 0
MAR_F32 = 0
MAR_BF16 = 1
MAR_CFG_STORE = 0
MAR_CFG_REUSE = 1
MAR_LAYER_CACHE = 1
MAR_LAYER_SELECT = 2
MAR_LAYER_GATE = 4
MAR_REFRESH_TOPK_SCRATCH_BYTES = 8 << 20


class MarError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class StepPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("step", "refresh", "gen_begin", "n_gen", "prev_begin", "n_prev", "n_refresh",
                 "n_active", "n_cached")]

    def as_dict(self):
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


_lib = None


def load_library(path: Optional[str] = None):
    """Load libmarca.so (built in-tree by __graft_entry__.build()); raises if missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else _LIB_PATH
    if not p.exists():
        raise ImportError(f"{p} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(str(p))
    V, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.mar_status_string.restype = ctypes.c_char_p
    lib.mar_status_string.argtypes = [I]
    lib.mar_version.restype = I
    lib.mar_cache_attn_fwd.restype = I
    lib.mar_cache_attn_fwd.argtypes = [V, V, V, V, V, V, I, V, V, I, I, I, I, I, I, F, I, V]
    lib.mar_cache_attn_fwd_ragged.restype = I
    lib.mar_cache_attn_fwd_ragged.argtypes = [V, V, V, V, V, V, I, V, V, V, V, I, I, I, I, I, I,
                                              F, I, V]
    lib.mar_cache_attn_fwd_update.restype = I
    lib.mar_cache_attn_fwd_update.argtypes = [V, V, V, V, V, V, I, V, I, V, V, V, I, I, I, I, I,
                                              I, F, I, V]
    lib.mar_cache_attn_fwd_ragged_update.restype = I
    lib.mar_cache_attn_fwd_ragged_update.argtypes = [V, V, V, V, V, V, I, V, I, V, V, V, V, V, I,
                                                     I, I, I, I, I, F, I, V]
    lib.mar_cache_attn_fwd_scores.restype = I
    lib.mar_cache_attn_fwd_scores.argtypes = [V, V, V, V, V, V, I, I, V, S, I, I, I, I, F, I, V]
    lib.mar_refresh_select.restype = I
    lib.mar_refresh_select.argtypes = [V, S, V, I, I, I, V, V, I, V, I, V, I, I, I, I, V]
    lib.mar_kv_scatter_refresh.restype = I
    lib.mar_kv_scatter_refresh.argtypes = [V, V, V, V, V, I, V, I, I, I, I, I, I, V]
    lib.mar_refresh_topk_workspace.restype = S
    lib.mar_refresh_topk_workspace.argtypes = [I, I, I]
    lib.mar_refresh_topk.restype = I
    lib.mar_refresh_topk.argtypes = [V, V, V, I, I, I, F, V, V, I, V, I, V, V, S, I, I, I, I, I,
                                     I, V]
    lib.mar_refresh_topk_noalloc.restype = I
    lib.mar_refresh_topk_noalloc.argtypes = [V, V, V, I, I, I, F, V, V, I, V, I, V, I, I, I, I,
                                             I, I, V]
    lib.mar_cos_gate.restype = I
    lib.mar_cos_gate.argtypes = [V, V, F, F, V, V, V, V, V, V, I, I, I, I, V]
    lib.mar_cfg_residual.restype = I
    lib.mar_cfg_residual.argtypes = [V, V, V, V, V, F, I, ctypes.c_int64, V]
    lib.mar_plan_step.restype = I
    lib.mar_plan_step.argtypes = [V, I, I, I, I, I, I, ctypes.POINTER(StepPlan)]
    lib.mar_layer_flags.restype = I
    lib.mar_layer_flags.argtypes = [ctypes.POINTER(StepPlan), I, I, I, I]
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != MAR_OK:
        raise MarError(fn, status, load_library().mar_status_string(status).decode())


_capture = None  # a list while prepare() records calls


def _call(name: str, *args, lib=None):
    """Call a device entry point with marshalled arguments (or record the call
    when prepare() is capturing) and raise MarError on a negative status."""
    fn = getattr(lib if lib is not None else load_library(), name)
    if _capture is not None:
        _capture.append((name, fn, args))
        return
    _check(name, fn(*args))


class Prepared:
    """Library calls whose arguments were checked and marshalled once: calling
    the object makes the same C calls again (same device pointers, sizes and
    stream), paying only for the foreign calls themselves."""

    def __init__(self, calls):
        self.calls = calls

    def __call__(self):
        for name, fn, args in self.calls:
            st = fn(*args)
            if st != MAR_OK:
                _check(name, st)


def prepare(fn, *args, **kwargs) -> Prepared:
    """Run the binding function fn(*args, **kwargs) once without executing its
    library calls: its checks and argument marshalling happen now (including
    the choice of stream, the current one unless given), and the returned
    Prepared replays the calls.  Every tensor it refers to must stay alive and
    in place while the Prepared is used; outputs fn would allocate are
    allocated once, here."""
    global _capture
    if _capture is not None:
        raise RuntimeError("prepare() does not nest")
    _capture = []
    try:
        fn(*args, **kwargs)
        calls = _capture
    finally:
        _capture = None
    return Prepared(calls)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MAR_F32
    if t.dtype == torch.bfloat16:
        return MAR_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def mar_cache_attn_fwd(q_a, k_a, v_a, k_cache, v_cache, cached_idx, Nc=None, out=None, lse=None,
                       scale=None, stream=None):
    """out [B,H,A,D] (and lse [B,H,A] when given) of cache-aware attention."""
    B, H, A, D = q_a.shape
    N = k_cache.shape[2]
    dt = q_a.dtype
    code = _dtype_code(q_a)
    for name, t in (("k_a", k_a), ("v_a", v_a)):
        _dev(t, name, dt, (B, H, A, D))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, dt, (B, H, N, D))
    if cached_idx is None:
        ldc, Nc = 0, 0 if Nc is None else Nc
        cptr = None
    else:
        if cached_idx.dim() != 2 or cached_idx.shape[0] != B:
            raise ValueError("cached_idx must be [B, ldc]")
        ldc = cached_idx.shape[1]
        Nc = ldc if Nc is None else int(Nc)
        cptr = _dev(cached_idx, "cached_idx", torch.int32)
    if out is None:
        out = torch.empty_like(q_a)
    _dev(out, "out", dt, (B, H, A, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, H, A))
    if scale is None:
        scale = D ** -0.5
    _call("mar_cache_attn_fwd",
        _dev(q_a, "q_a"), _dev(k_a, "k_a"), _dev(v_a, "v_a"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), cptr, ldc, _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else None, B, H, N, A, Nc, D, float(scale), code,
        _stream(stream))
    return out


def mar_cache_attn_fwd_ragged(q_a, k_a, v_a, k_cache, v_cache, cached_idx, a_len, c_len,
                              out=None, lse=None, scale=None, stream=None):
    """mar_cache_attn_fwd with per-sequence counts: a_len [B] active rows (of the A
    row capacity), c_len [B] cached entries (of cached_idx's ldc columns).  Rows
    past a sequence's count are not written (out is zero-filled when allocated here)."""
    B, H, A, D = q_a.shape
    N = k_cache.shape[2]
    dt = q_a.dtype
    code = _dtype_code(q_a)
    for name, t in (("k_a", k_a), ("v_a", v_a)):
        _dev(t, name, dt, (B, H, A, D))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, dt, (B, H, N, D))
    if cached_idx is None:
        ldc, cptr = 0, None
    else:
        if cached_idx.dim() != 2 or cached_idx.shape[0] != B:
            raise ValueError("cached_idx must be [B, ldc]")
        ldc = cached_idx.shape[1]
        cptr = _dev(cached_idx, "cached_idx", torch.int32)
    for name, t in (("a_len", a_len), ("c_len", c_len)):
        _dev(t, name, torch.int32, (B,))
    if out is None:
        out = torch.zeros_like(q_a)
    _dev(out, "out", dt, (B, H, A, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, H, A))
    if scale is None:
        scale = D ** -0.5
    _call("mar_cache_attn_fwd_ragged",
        _dev(q_a, "q_a"), _dev(k_a, "k_a"), _dev(v_a, "v_a"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), cptr, ldc, _dev(a_len, "a_len"), _dev(c_len, "c_len"),
        _dev(out, "out"), _dev(lse, "lse") if lse is not None else None, B, H, N, A, ldc, D,
        float(scale), code, _stream(stream))
    return out


def mar_cache_attn_fwd_ragged_update(q_a, k_a, v_a, k_cache, v_cache, cached_idx, active_idx,
                                     a_len, c_len, out=None, lse=None, err_count=None, scale=None,
                                     stream=None):
    """mar_cache_attn_fwd_ragged, plus each sequence's first a_len[b] rows of
    k_a/v_a written into k_cache/v_cache at active_idx [B, ld] (entries at or
    past a_len[b] are not read) in the same pass.  Returns out."""
    B, H, A, D = q_a.shape
    N = k_cache.shape[2]
    dt = q_a.dtype
    code = _dtype_code(q_a)
    for name, t in (("k_a", k_a), ("v_a", v_a)):
        _dev(t, name, dt, (B, H, A, D))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, dt, (B, H, N, D))
    if cached_idx is None:
        ldc, cptr = 0, None
    else:
        if cached_idx.dim() != 2 or cached_idx.shape[0] != B:
            raise ValueError("cached_idx must be [B, ldc]")
        ldc = cached_idx.shape[1]
        cptr = _dev(cached_idx, "cached_idx", torch.int32)
    if active_idx.dim() != 2 or active_idx.shape[0] != B:
        raise ValueError("active_idx must be [B, ld_act]")
    for name, t in (("a_len", a_len), ("c_len", c_len)):
        _dev(t, name, torch.int32, (B,))
    if out is None:
        out = torch.zeros_like(q_a)
    _dev(out, "out", dt, (B, H, A, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, H, A))
    if scale is None:
        scale = D ** -0.5
    _call("mar_cache_attn_fwd_ragged_update",
        _dev(q_a, "q_a"), _dev(k_a, "k_a"), _dev(v_a, "v_a"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), cptr, ldc, _dev(active_idx, "active_idx", torch.int32),
        active_idx.shape[1], _dev(a_len, "a_len"), _dev(c_len, "c_len"),
        _dev(err_count, "err_count", torch.int32), _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else None, B, H, N, A, ldc, D, float(scale), code,
        _stream(stream))
    return out


def mar_cache_attn_fwd_update(q_a, k_a, v_a, k_cache, v_cache, cached_idx, active_idx, Nc=None,
                              out=None, lse=None, err_count=None, scale=None, stream=None):
    """mar_cache_attn_fwd, plus k_cache/v_cache rows at active_idx [B, ld] (first A
    entries) overwritten with k_a/v_a in the same pass.  active_idx None is the full
    refresh (A == N, no cached rows): the caches become k_a/v_a.  Returns out."""
    B, H, A, D = q_a.shape
    N = k_cache.shape[2]
    dt = q_a.dtype
    code = _dtype_code(q_a)
    for name, t in (("k_a", k_a), ("v_a", v_a)):
        _dev(t, name, dt, (B, H, A, D))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, dt, (B, H, N, D))
    if cached_idx is None:
        ldc, Nc = 0, 0 if Nc is None else Nc
        cptr = None
    else:
        if cached_idx.dim() != 2 or cached_idx.shape[0] != B:
            raise ValueError("cached_idx must be [B, ldc]")
        ldc = cached_idx.shape[1]
        Nc = ldc if Nc is None else int(Nc)
        cptr = _dev(cached_idx, "cached_idx", torch.int32)
    if active_idx is None:
        ld_act, aptr = 0, None
    else:
        if active_idx.dim() != 2 or active_idx.shape[0] != B or active_idx.stride(1) != 1:
            raise ValueError("active_idx must be [B, ld] with unit column stride")
        ld_act = active_idx.stride(0)
        aptr = ctypes.c_void_p(active_idx.data_ptr())
        if active_idx.dtype != torch.int32 or not active_idx.is_cuda:
            raise ValueError("active_idx must be an int32 device tensor")
    if out is None:
        out = torch.empty_like(q_a)
    _dev(out, "out", dt, (B, H, A, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, H, A))
    if err_count is not None:
        _dev(err_count, "err_count", torch.int32)
    if scale is None:
        scale = D ** -0.5
    _call("mar_cache_attn_fwd_update",
        _dev(q_a, "q_a"), _dev(k_a, "k_a"), _dev(v_a, "v_a"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), cptr, ldc, aptr, ld_act,
        _dev(err_count, "err_count") if err_count is not None else None, _dev(out, "out"),
        _dev(lse, "lse") if lse is not None else None, B, H, N, A, Nc, D, float(scale), code,
        _stream(stream))
    return out


def mar_kv_scatter_refresh(k_cache, v_cache, k_new, v_new, idx=None, err_count=None, stream=None):
    """In-place cache update at idx [B, ld] (first M entries), or full copy when idx is None."""
    B, H, N, D = k_cache.shape
    M = k_new.shape[2]
    dt = k_cache.dtype
    code = _dtype_code(k_cache)
    _dev(v_cache, "v_cache", dt, (B, H, N, D))
    _dev(k_new, "k_new", dt, (B, H, M, D))
    _dev(v_new, "v_new", dt, (B, H, M, D))
    ld = 0
    if idx is not None:
        if idx.dim() != 2 or idx.shape[0] != B:
            raise ValueError("idx must be [B, ld_idx]")
        ld = idx.shape[1]
    _call("mar_kv_scatter_refresh",
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_new, "k_new"),
        _dev(v_new, "v_new"), _dev(idx, "idx", torch.int32), ld,
        _dev(err_count, "err_count", torch.int32), B, H, N, M, D, code, _stream(stream))


def mar_refresh_topk_workspace(B: int, H: int, N: int) -> int:
    return int(load_library().mar_refresh_topk_workspace(B, H, N))


def mar_refresh_topk(q_gen, k_full, gp_idx, n_gp, K, scores=None, active_idx=None,
                     cached_idx=None, cached_len=None, workspace=None, scale=None, stream=None,
                     _noalloc=False):
    """Returns (scores [B,N], active_idx [B,ld_act], cached_idx [B,ld_cached], cached_len [B]).
    With _noalloc the call goes to mar_refresh_topk_noalloc (no workspace)."""
    B, H, G, D = q_gen.shape
    N = k_full.shape[2]
    dt = q_gen.dtype
    code = _dtype_code(q_gen)
    _dev(k_full, "k_full", dt, (B, H, N, D))
    dev = q_gen.device
    if gp_idx is None:
        ld_gp = 0
    else:
        if gp_idx.dim() != 2 or gp_idx.shape[0] != B:
            raise ValueError("gp_idx must be [B, ld_gp]")
        ld_gp = gp_idx.stride(0)
        if gp_idx.stride(1) != 1:
            raise ValueError("gp_idx rows must be contiguous")
    if scores is None:
        scores = torch.empty((B, N), dtype=torch.float32, device=dev)
    if active_idx is None:
        active_idx = torch.empty((B, max(n_gp + K, 1)), dtype=torch.int32, device=dev)
    if cached_idx is None:
        cached_idx = torch.empty((B, N), dtype=torch.int32, device=dev)
    if cached_len is None:
        cached_len = torch.empty((B,), dtype=torch.int32, device=dev)
    ws_bytes = mar_refresh_topk_workspace(B, H, N)
    if workspace is None and not _noalloc:
        workspace = torch.empty((ws_bytes // 4,), dtype=torch.float32, device=dev)
    _dev(scores, "scores", torch.float32, (B, N))
    _dev(cached_len, "cached_len", torch.int32, (B,))
    gp_ptr = None
    if gp_idx is not None:
        if not gp_idx.is_cuda or gp_idx.dtype != torch.int32:
            raise ValueError("gp_idx must be a GPU int32 tensor")
        gp_ptr = ctypes.c_void_p(gp_idx.data_ptr())
    if _noalloc:
        _call("mar_refresh_topk_noalloc",
            _dev(q_gen, "q_gen"), _dev(k_full, "k_full"), gp_ptr, ld_gp, int(n_gp), int(K),
            float(D ** -0.5 if scale is None else scale), _dev(scores, "scores"),
            _dev(active_idx, "active_idx", torch.int32), active_idx.shape[1],
            _dev(cached_idx, "cached_idx", torch.int32), cached_idx.shape[1],
            _dev(cached_len, "cached_len"), B, H, G, N, D, code, _stream(stream))
        return scores, active_idx, cached_idx, cached_len
    _call("mar_refresh_topk",
        _dev(q_gen, "q_gen"), _dev(k_full, "k_full"), gp_ptr, ld_gp, int(n_gp), int(K),
        float(D ** -0.5 if scale is None else scale), _dev(scores, "scores"),
        _dev(active_idx, "active_idx", torch.int32), active_idx.shape[1],
        _dev(cached_idx, "cached_idx", torch.int32), cached_idx.shape[1],
        _dev(cached_len, "cached_len"), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), B, H, G, N, D, code, _stream(stream))
    return scores, active_idx, cached_idx, cached_len


def mar_cache_attn_fwd_scores(q, k, v, gen_idx, G, partials=None, out=None, lse=None,
                              scale=None, stream=None):
    """Layer 2's full attention over all N tokens that also writes the per-head
    sums of the G generating queries' probabilities (see mar_cache_attn.h).
    gen_idx [B, ld_gen] int32.  Returns (out [B,H,N,D], partials [B,H,N] float32)."""
    B, H, N, D = q.shape
    dt = q.dtype
    for name, t in (("k", k), ("v", v)):
        _dev(t, name, dt, (B, H, N, D))
    if gen_idx.dim() != 2 or gen_idx.shape[0] != B or gen_idx.stride(1) != 1:
        raise ValueError("gen_idx must be [B, ld_gen] with contiguous rows")
    if not gen_idx.is_cuda or gen_idx.dtype != torch.int32:
        raise ValueError("gen_idx must be a GPU int32 tensor")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", dt, (B, H, N, D))
    if partials is None:
        partials = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _dev(partials, "partials", torch.float32, (B, H, N))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, H, N))
    _call("mar_cache_attn_fwd_scores", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
          _dev(lse, "lse") if lse is not None else None, ctypes.c_void_p(gen_idx.data_ptr()),
          gen_idx.stride(0), int(G), _dev(partials, "partials"), partials.numel() * 4, B, H, N, D,
          float(D ** -0.5 if scale is None else scale), _dtype_code(q), _stream(stream))
    return out, partials


def mar_refresh_select(partials, gp_idx, n_gp, K, G, scores=None, active_idx=None,
                       cached_idx=None, cached_len=None, stream=None):
    """The selection half of mar_refresh_topk from per-head partials [B,H,N]
    (mar_cache_attn_fwd_scores writes them).  Returns (scores, active_idx,
    cached_idx, cached_len) as mar_refresh_topk does."""
    B, H, N = partials.shape
    _dev(partials, "partials", torch.float32, (B, H, N))
    dev = partials.device
    if gp_idx is None:
        ld_gp, gp_ptr = 0, None
    else:
        if gp_idx.dim() != 2 or gp_idx.shape[0] != B or gp_idx.stride(1) != 1:
            raise ValueError("gp_idx must be [B, ld_gp] with contiguous rows")
        if not gp_idx.is_cuda or gp_idx.dtype != torch.int32:
            raise ValueError("gp_idx must be a GPU int32 tensor")
        ld_gp, gp_ptr = gp_idx.stride(0), ctypes.c_void_p(gp_idx.data_ptr())
    if scores is None:
        scores = torch.empty((B, N), dtype=torch.float32, device=dev)
    if active_idx is None:
        active_idx = torch.empty((B, max(n_gp + K, 1)), dtype=torch.int32, device=dev)
    if cached_idx is None:
        cached_idx = torch.empty((B, N), dtype=torch.int32, device=dev)
    if cached_len is None:
        cached_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _dev(scores, "scores", torch.float32, (B, N))
    _dev(cached_len, "cached_len", torch.int32, (B,))
    _call("mar_refresh_select", _dev(partials, "partials"), partials.numel() * 4, gp_ptr, ld_gp,
          int(n_gp), int(K), _dev(scores, "scores"),
          _dev(active_idx, "active_idx", torch.int32), active_idx.shape[1],
          _dev(cached_idx, "cached_idx", torch.int32), cached_idx.shape[1],
          _dev(cached_len, "cached_len"), B, H, int(G), N, _stream(stream))
    return scores, active_idx, cached_idx, cached_len


def mar_refresh_topk_noalloc(q_gen, k_full, gp_idx, n_gp, K, scores=None, active_idx=None,
                             cached_idx=None, cached_len=None, scale=None, stream=None):
    """mar_refresh_topk through the allocation-free entry point: the library's
    per-device array takes the partial scores.  Output tensors left as None
    are allocated here by torch (pass them in to allocate nothing)."""
    return mar_refresh_topk(q_gen, k_full, gp_idx, n_gp, K, scores, active_idx, cached_idx,
                            cached_len, None, scale, stream, _noalloc=True)


def mar_cos_gate(x_cur, x_cached, tau=0.95, eps=1e-8, cos_out=None, reuse_mask=None,
                 compute_idx=None, compute_len=None, reuse_idx=None, reuse_len=None,
                 stream=None):
    """Returns (cos [B,N] f32, reuse [B,N] u8, compute_idx [B,N] i32, compute_len [B] i32).
    With reuse_idx [B,N] i32 and reuse_len [B] i32 given (both or neither),
    also fills the ascending reusing positions (-1 padded) and their counts."""
    B, N, W = x_cur.shape
    code = _dtype_code(x_cur)
    _dev(x_cached, "x_cached", x_cur.dtype, (B, N, W))
    dev = x_cur.device
    if cos_out is None:
        cos_out = torch.empty((B, N), dtype=torch.float32, device=dev)
    if reuse_mask is None:
        reuse_mask = torch.empty((B, N), dtype=torch.uint8, device=dev)
    if compute_idx is None:
        compute_idx = torch.empty((B, N), dtype=torch.int32, device=dev)
    if compute_len is None:
        compute_len = torch.empty((B,), dtype=torch.int32, device=dev)
    _call("mar_cos_gate",
        _dev(x_cur, "x_cur"), _dev(x_cached, "x_cached"), float(tau), float(eps),
        _dev(cos_out, "cos_out", torch.float32, (B, N)),
        _dev(reuse_mask, "reuse_mask", torch.uint8, (B, N)),
        _dev(compute_idx, "compute_idx", torch.int32, (B, N)),
        _dev(compute_len, "compute_len", torch.int32, (B,)),
        None if reuse_idx is None else _dev(reuse_idx, "reuse_idx", torch.int32, (B, N)),
        None if reuse_len is None else _dev(reuse_len, "reuse_len", torch.int32, (B,)),
        B, N, W, code, _stream(stream))
    return cos_out, reuse_mask, compute_idx, compute_len


def mar_cfg_residual(cond, uncond=None, residual=None, mode=MAR_CFG_STORE, uncond_out=None,
                     guided_out=None, cfg_scale=1.0, stream=None):
    """STORE: fills residual (allocated if None); REUSE: fills uncond_out.  Returns the outputs."""
    f32 = torch.float32
    _dev(cond, "cond", f32)
    n = cond.numel()
    if mode == MAR_CFG_STORE:
        _dev(uncond, "uncond", f32, cond.shape)
        if residual is None:
            residual = torch.empty_like(cond)
    else:
        if uncond_out is None:
            uncond_out = torch.empty_like(cond)
        _dev(uncond_out, "uncond_out", f32, cond.shape)
    _dev(residual, "residual", f32, cond.shape)
    if guided_out is not None:
        _dev(guided_out, "guided_out", f32, cond.shape)
    _call("mar_cfg_residual",
        _dev(cond, "cond"), _dev(uncond, "uncond") if uncond is not None else None,
        _dev(residual, "residual"), _dev(uncond_out, "uncond_out") if uncond_out is not None else None,
        _dev(guided_out, "guided_out") if guided_out is not None else None, float(cfg_scale),
        int(mode), n, _stream(stream))
    return (residual if mode == MAR_CFG_STORE else uncond_out), guided_out


def mar_plan_step(counts, step: int, n_tokens: int, budget: int, period: int = 3,
                  warmup: int = 0) -> StepPlan:
    """Host-side step plan (no GPU).  counts: sequence of per-step token counts."""
    arr = (ctypes.c_int32 * len(counts))(*[int(c) for c in counts])
    plan = StepPlan()
    st = load_library().mar_plan_step(ctypes.cast(arr, ctypes.c_void_p), len(counts), int(step),
                                      int(n_tokens), int(budget), int(period), int(warmup),
                                      ctypes.byref(plan))
    _check("mar_plan_step", st)
    return plan


def mar_layer_flags(plan: StepPlan, layer: int, n_full_layers: int = 2, select_layer: int = 2,
                    ungated_layers: int = 3) -> int:
    r = load_library().mar_layer_flags(ctypes.byref(plan), int(layer), int(n_full_layers),
                                       int(select_layer), int(ungated_layers))
    if r < 0:
        _check("mar_layer_flags", r)
    return r
