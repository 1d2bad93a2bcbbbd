"""CPU oracle for the KV-cached MAR decoding hot path.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  Nothing here imports the GPU package
and the GPU package never imports this one; they share no code.

The arithmetic lives in ``oracle.c`` (plain scalar C, double precision); this
module only compiles it with gcc when needed and marshals numpy arrays into it.
The schedule logic (pure integers) is in ``schedule.py``.

Pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_HDR = _HERE / "oracle.h"
_LIB = _HERE / "liboracle.so"

_lib = None


def build(force: bool = False) -> Path:
    """Compile liboracle.so with gcc (OpenMP) if missing or older than its sources."""
    newest = max(_SRC.stat().st_mtime, _HDR.stat().st_mtime)
    if force or not _LIB.exists() or _LIB.stat().st_mtime < newest:
        tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
               "-Wall", "-Wextra", "-o", str(tmp), str(_SRC), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    lib = ctypes.CDLL(str(build()))
    P = ctypes.c_void_p
    I = ctypes.c_int64
    D = ctypes.c_double
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_cache_attention.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, P]
    lib.oracle_cache_attention.restype = ctypes.c_int
    lib.oracle_refresh_scores.argtypes = [P, P, I, I, I, I, I, D, P]
    lib.oracle_refresh_select.argtypes = [P, P, I, I, I, I, I, P, I, P, I, P]
    lib.oracle_kv_scatter.argtypes = [P, P, P, P, P, I, I, I, I, I, I]
    lib.oracle_kv_scatter.restype = ctypes.c_int64
    lib.oracle_cos_gate.argtypes = [P, P, I, I, I, D, D, P, P, P, P]
    lib.oracle_gate_from_cos.argtypes = [P, I, I, D, P, P, P]
    lib.oracle_cfg_residual.argtypes = [P, P, P, P, P, D, ctypes.c_int, I]
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def cache_attention(q_a, k_a, v_a, k_cache, v_cache, cached_idx, scale, Nc=None):
    """Attention of the active queries over [K_A ; K_cache[cached_idx]].

    q_a,k_a,v_a: [B,H,A,D]; k_cache,v_cache: [B,H,N,D]; cached_idx: [B,ldc]
    (first Nc entries used; Nc defaults to ldc).  Returns (out [B,H,A,D], lse [B,H,A]).
    """
    q_a, k_a, v_a = _f64(q_a), _f64(k_a), _f64(v_a)
    k_cache, v_cache = _f64(k_cache), _f64(v_cache)
    cached_idx = _i32(cached_idx)
    B, H, A, D = q_a.shape
    N = k_cache.shape[2]
    ldc = cached_idx.shape[1] if cached_idx.ndim == 2 else 0
    Nc = ldc if Nc is None else int(Nc)
    if cached_idx.size == 0:
        cached_idx = np.zeros((B, 1), np.int32)
        ldc = 1
    out = np.empty((B, H, A, D), np.float64)
    lse = np.empty((B, H, A), np.float64)
    rc = _load().oracle_cache_attention(_p(q_a), _p(k_a), _p(v_a), _p(k_cache), _p(v_cache),
                                        _p(cached_idx), ldc, B, H, N, A, Nc, D, float(scale),
                                        _p(out), _p(lse))
    if rc != 0:
        raise ValueError("cached index out of range")
    return out, lse


def refresh_scores(q_gen, k_full, scale):
    """[B,N] mean over heads and generating queries of the full-attention rows."""
    q_gen, k_full = _f64(q_gen), _f64(k_full)
    B, H, G, D = q_gen.shape
    N = k_full.shape[2]
    scores = np.empty((B, N), np.float64)
    _load().oracle_refresh_scores(_p(q_gen), _p(k_full), B, H, G, N, D, float(scale), _p(scores))
    return scores


def refresh_select(scores, gp_idx, K, ld_cached=None):
    """Top-K over non-G/P tokens (score desc, index asc) + ascending complement.

    Returns (active_idx [B, n_gp+K], cached_idx [B, ld_cached], cached_len [B]).
    """
    scores = _f64(scores)
    gp_idx = _i32(gp_idx)
    B, N = scores.shape
    n_gp = gp_idx.shape[1]
    if gp_idx.size == 0:
        gp_idx = np.zeros((B, 1), np.int32)
    ld_gp = gp_idx.shape[1]
    ld_act = max(n_gp + K, 1)
    ld_cached = N if ld_cached is None else int(ld_cached)
    active = np.empty((B, ld_act), np.int32)
    cached = np.empty((B, max(ld_cached, 1)), np.int32)
    clen = np.empty((B,), np.int32)
    _load().oracle_refresh_select(_p(scores), _p(gp_idx), ld_gp, n_gp, int(K), B, N,
                                  _p(active), ld_act, _p(cached), max(ld_cached, 1), _p(clen))
    return active[:, :n_gp + K], cached[:, :ld_cached], clen


def kv_scatter(k_cache, v_cache, k_new, v_new, idx):
    """Returns (k_cache', v_cache', skipped) computed on copies of the raw bytes."""
    kc = np.ascontiguousarray(np.array(k_cache, copy=True))
    vc = np.ascontiguousarray(np.array(v_cache, copy=True))
    kn = np.ascontiguousarray(k_new)
    vn = np.ascontiguousarray(v_new)
    assert kc.dtype == kn.dtype == vc.dtype == vn.dtype
    B, H, N, D = kc.shape
    M = kn.shape[2]
    if idx is None:
        assert M == N
        ip = None
    else:
        idx = _i32(idx)
        ip = _p(idx)
    skipped = _load().oracle_kv_scatter(_p(kc), _p(vc), _p(kn), _p(vn), ip, B, H, N, M, D,
                                        kc.dtype.itemsize)
    return kc, vc, int(skipped)


def cos_gate(x, y, tau, eps=1e-8):
    """Returns (cos [B,N], reuse [B,N] u8, compute_idx [B,N], compute_len [B])."""
    x, y = _f64(x), _f64(y)
    B, N, W = x.shape
    cos = np.empty((B, N), np.float64)
    reuse = np.empty((B, N), np.uint8)
    cidx = np.empty((B, N), np.int32)
    clen = np.empty((B,), np.int32)
    _load().oracle_cos_gate(_p(x), _p(y), B, N, W, float(tau), float(eps), _p(cos), _p(reuse),
                            _p(cidx), _p(clen))
    return cos, reuse, cidx, clen


def gate_from_cos(cos, tau):
    """Mask and compaction from given cosines (decision on exactly those values)."""
    cos = _f64(cos)
    B, N = cos.shape
    reuse = np.empty((B, N), np.uint8)
    cidx = np.empty((B, N), np.int32)
    clen = np.empty((B,), np.int32)
    _load().oracle_gate_from_cos(_p(cos), B, N, float(tau), _p(reuse), _p(cidx), _p(clen))
    return reuse, cidx, clen


def cfg_residual(cond, uncond=None, residual=None, mode=0, w=None):
    """mode 0: returns (residual, guided|None); mode 1: returns (uncond_out, guided|None)."""
    cond = np.ascontiguousarray(cond, dtype=np.float32)
    n = cond.size
    guided = np.empty_like(cond) if w is not None else None
    gp = _p(guided) if guided is not None else None
    if mode == 0:
        uncond = np.ascontiguousarray(uncond, dtype=np.float32)
        res = np.empty_like(cond)
        _load().oracle_cfg_residual(_p(cond), _p(uncond), _p(res), None, gp,
                                    float(w or 0.0), 0, n)
        return res, guided
    residual = np.ascontiguousarray(residual, dtype=np.float32)
    uo = np.empty_like(cond)
    _load().oracle_cfg_residual(_p(cond), None, _p(residual), _p(uo), gp, float(w or 0.0), 1, n)
    return uo, guided
