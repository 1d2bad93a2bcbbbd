"""ctypes binding of libmarca_bench (include/mar_bench.h): measurement kernels
used by the benchmark, not part of the decoding path.  Argument marshalling
only, as in _lib; the calls can be prepared with _lib.prepare."""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

from ._lib import MAR_BF16, _call, _dev, _dtype_code, _stream

_PATH = Path(__file__).resolve().parent / "libmarca_bench.so"
_blib = None


def load_bench_library():
    global _blib
    if _blib is None:
        if not _PATH.exists():
            raise ImportError(f"{_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
                              "g.build()'`")
        lib = ctypes.CDLL(str(_PATH))
        V, I = ctypes.c_void_p, ctypes.c_int
        lib.mar_bench_attn_pattern.restype = I
        lib.mar_bench_attn_pattern.argtypes = [V, V, V, V, V, V, I, V, I, I, I, I, I, I, I, I, V]
        lib.mar_bench_kv_concat.restype = I
        lib.mar_bench_kv_concat.argtypes = [V, V, V, V, V, V, V, I, I, I, I, I, I, I, I, V]
        lib.mar_bench_dense_floor.restype = I
        lib.mar_bench_dense_floor.argtypes = [V, V, V, V, V, V, I, I, I, I, I, I, V]
        lib.mar_bench_cached_floor.restype = I
        lib.mar_bench_cached_floor.argtypes = [V, V, V, V, V, V, I, V, I, V, V, V, I, I, I, I,
                                               I, I, I, I, V]
        _blib = lib
    return _blib


def mar_bench_attn_pattern(q_a, k_a, v_a, k_cache, v_cache, cached_idx, Nc, out, write_out=True,
                           stream=None):
    """The attention's memory operations without its arithmetic (see mar_bench.h)."""
    B, H, A, D = q_a.shape
    N = k_cache.shape[2]
    dt = q_a.dtype
    for name, t in (("k_a", k_a), ("v_a", v_a), ("out", out)):
        _dev(t, name, dt, (B, H, A, D))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, dt, (B, H, N, D))
    _call("mar_bench_attn_pattern", _dev(q_a, "q_a"), _dev(k_a, "k_a"), _dev(v_a, "v_a"),
          _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
          _dev(cached_idx, "cached_idx", torch.int32), cached_idx.shape[1], _dev(out, "out"),
          int(bool(write_out)), B, H, N, A, int(Nc), D, _dtype_code(q_a), _stream(stream),
          lib=load_bench_library())
    return out


MAR_BENCH_FLOOR_ARITH = 1
MAR_BENCH_FLOOR_MEMORY = 2


def mar_bench_dense_floor(q, k, v, out, mode, k_cache=None, v_cache=None, stream=None):
    """The full-attention kernel's arithmetic alone (MAR_BENCH_FLOOR_ARITH) or
    its memory operations alone (MAR_BENCH_FLOOR_MEMORY) over q, k, v, out
    [B,H,N,D]; with k_cache, v_cache [B,H,N,D] the refresh-step layer's (see
    mar_bench.h)."""
    B, H, N, D = q.shape
    for name, t in (("k", k), ("v", v), ("out", out)):
        _dev(t, name, q.dtype, (B, H, N, D))
    caches = []
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        caches.append(None if t is None else _dev(t, name, q.dtype, (B, H, N, D)))
    _call("mar_bench_dense_floor", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), caches[0],
          caches[1], _dev(out, "out"), int(mode), B, H, N, D, _dtype_code(q), _stream(stream),
          lib=load_bench_library())
    return out


def mar_bench_cached_floor(q_a, k_a, v_a, k_cache, v_cache, cached_idx, out, mode, Nc=None,
                           active_idx=None, a_len=None, c_len=None, stream=None):
    """The cached workgroup kernel's arithmetic alone (MAR_BENCH_FLOOR_ARITH)
    or its memory operations alone (MAR_BENCH_FLOOR_MEMORY): the layer of
    mar_cache_attn_fwd (Nc cached entries, default all of cached_idx's
    columns), or with active_idx, a_len, c_len that of
    mar_cache_attn_fwd_ragged_update (see mar_bench.h)."""
    B, H, A, D = q_a.shape
    N = k_cache.shape[2]
    dt = q_a.dtype
    for name, t in (("k_a", k_a), ("v_a", v_a), ("out", out)):
        _dev(t, name, dt, (B, H, A, D))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, dt, (B, H, N, D))
    if cached_idx.dim() != 2 or cached_idx.shape[0] != B:
        raise ValueError("cached_idx must be [B, ldc]")
    ldc = cached_idx.shape[1]
    aptr, ld_act = None, 0
    if active_idx is not None:
        if active_idx.dim() != 2 or active_idx.shape[0] != B:
            raise ValueError("active_idx must be [B, ld_act]")
        aptr, ld_act = _dev(active_idx, "active_idx", torch.int32), active_idx.shape[1]
    lens = [None if t is None else _dev(t, name, torch.int32, (B,))
            for name, t in (("a_len", a_len), ("c_len", c_len))]
    _call("mar_bench_cached_floor", _dev(q_a, "q_a"), _dev(k_a, "k_a"), _dev(v_a, "v_a"),
          _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
          _dev(cached_idx, "cached_idx", torch.int32), ldc, aptr, ld_act, lens[0], lens[1],
          _dev(out, "out"), int(mode), B, H, N, A, ldc if Nc is None else int(Nc), D,
          _dtype_code(q_a), _stream(stream), lib=load_bench_library())
    return out


def mar_bench_kv_concat(k_a, v_a, k_cache, v_cache, cached_idx, Nc, k_cat=None, v_cat=None,
                        stream=None):
    """[active rows ; cached rows] as contiguous [B,H,A+Nc,D] tensors (see mar_bench.h)."""
    B, H, A, D = k_a.shape
    N = k_cache.shape[2]
    dt = k_a.dtype
    T = A + int(Nc)
    if k_cat is None:
        k_cat = torch.empty((B, H, T, D), dtype=dt, device=k_a.device)
    if v_cat is None:
        v_cat = torch.empty_like(k_cat)
    for name, t in (("k_cat", k_cat), ("v_cat", v_cat)):
        _dev(t, name, dt, (B, H, T, D))
    _dev(v_a, "v_a", dt, (B, H, A, D))
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, dt, (B, H, N, D))
    _call("mar_bench_kv_concat", _dev(k_cat, "k_cat"), _dev(v_cat, "v_cat"), _dev(k_a, "k_a"),
          _dev(v_a, "v_a"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
          _dev(cached_idx, "cached_idx", torch.int32), cached_idx.shape[1], B, H, N, A, int(Nc),
          D, _dtype_code(k_a), _stream(stream), lib=load_bench_library())
    return k_cat, v_cat
