"""Host-side checks of libmarca's C ABI (no GPU needed).

The library must load, export every function include/mar_cache_attn.h
declares, reject bad arguments with the documented status before any GPU work,
and its host step planner must agree with the oracle's schedule.
"""
import ctypes
import os
import re

import pytest

from cache_aware_attention_amd import _lib
from mar_workloads import CONFIGS, cosine_counts
from oracle import schedule as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mar_cache_attn.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_RANGE, E_WS, E_LAUNCH, E_UNSUP = 0, -1, -2, -3, -4, -5, -6, -7
P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced (calls fail first)
BAD = 0x10008  # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mar_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 10
    raw = ctypes.CDLL(str(_lib._LIB_PATH))
    for n in names:
        assert hasattr(raw, n), f"{n} not exported"


def test_bench_library_exports_and_rejections():
    """libmarca_bench (include/mar_bench.h, measurement kernels) exports what it
    declares and refuses bad arguments before any GPU work."""
    from cache_aware_attention_amd import _bench_lib
    names = declared_functions(os.path.join(ROOT, "include", "mar_bench.h"))
    assert names == ["mar_bench_attn_pattern", "mar_bench_cached_floor", "mar_bench_dense_floor",
                     "mar_bench_kv_concat"]
    b = _bench_lib.load_bench_library()
    for n in names:
        assert hasattr(ctypes.CDLL(str(_bench_lib._PATH)), n)
    f = b.mar_bench_attn_pattern
    # q, ka, va, kc, vc, cidx, ldc, out, write, B, H, N, A, Nc, D, dtype, stream
    assert f(None, P, P, P, P, P, 272, P, 1, 2, 2, 320, 48, 272, 64, 1, None) == E_NULL
    assert f(P, P, P, P, P, P, 272, P, 1, 2, 2, 320, 48, 272, 64, 0, None) == E_UNSUP   # fp32
    assert f(P, P, P, P, P, P, 272, P, 1, 2, 2, 320, 49, 272, 64, 1, None) == E_SHAPE   # A+Nc > N
    assert f(P, P, P, P, P, P, 272, P, 1, 2, 2, 400, 80, 272, 64, 1, None) == E_UNSUP   # A > 64
    assert f(P, P, P, P, P, P, 100, P, 1, 2, 2, 320, 48, 272, 64, 1, None) == E_SHAPE   # ldc < Nc
    assert f(P, P, P, P, P, P, 272, BAD, 1, 2, 2, 320, 48, 272, 64, 1, None) == E_RANGE
    g = b.mar_bench_kv_concat
    # kcat, vcat, ka, va, kc, vc, cidx, ldc, B, H, N, A, Nc, D, dtype, stream
    assert g(None, P, P, P, P, P, P, 272, 2, 2, 320, 48, 272, 64, 1, None) == E_NULL
    assert g(P, P, P, P, P, P, P, 272, 2, 2, 320, 48, 272, 64, 7, None) == E_DTYPE
    assert g(P, P, P, P, P, P, P, 272, 2, 2, 320, 48, 272, 12, 1, None) == E_UNSUP    # 24-byte rows
    assert g(P, P, P, P, P, P, P, 100, 2, 2, 320, 48, 272, 64, 1, None) == E_SHAPE
    d = b.mar_bench_dense_floor
    # q, k, v, kc, vc, out, mode, B, H, N, D, dtype, stream
    assert d(None, P, P, None, None, P, 1, 2, 2, 320, 64, 1, None) == E_NULL
    assert d(P, P, P, P, None, P, 1, 2, 2, 320, 64, 1, None) == E_NULL      # one cache only
    assert d(P, P, P, None, None, P, 1, 2, 2, 320, 64, 0, None) == E_UNSUP  # fp32
    assert d(P, P, P, None, None, P, 1, 0, 2, 320, 64, 1, None) == E_SHAPE
    assert d(P, P, P, None, None, P, 1, 2, 2, 64, 64, 1, None) == E_UNSUP   # one wave's tokens
    assert d(P, P, P, None, None, P, 1, 2, 2, 320, 32, 1, None) == E_UNSUP  # head dim
    assert d(P, P, P, None, None, P, 3, 2, 2, 320, 64, 1, None) == E_RANGE  # no such mode
    assert d(P, P, P, None, None, BAD, 2, 2, 2, 320, 64, 1, None) == E_RANGE
    assert d(P, P, P, BAD, P, P, 2, 2, 2, 320, 64, 1, None) == E_RANGE
    c = b.mar_bench_cached_floor
    # q, ka, va, kc, vc, cidx, ldc, act, ld_act, a_len, c_len, out, mode, B, H, N, A, Nc, D,
    # dtype, stream
    assert c(P, P, P, P, P, None, 960, None, 0, None, None, P, 1, 2, 2, 1088, 128, 960, 64, 1,
             None) == E_NULL
    assert c(P, P, P, P, P, P, 1088, P, 200, P, None, P, 1, 2, 2, 1088, 200, 1088, 64, 1,
             None) == E_NULL                                                     # a_len only
    assert c(P, P, P, P, P, P, 960, P, 128, None, None, P, 1, 2, 2, 1088, 128, 960, 64, 1,
             None) == E_UNSUP                                                    # uniform update
    assert c(P, P, P, P, P, P, 960, None, 0, None, None, P, 1, 2, 2, 1088, 128, 960, 64, 0,
             None) == E_UNSUP                                                    # fp32
    assert c(P, P, P, P, P, P, 961, None, 0, None, None, P, 1, 2, 2, 1088, 128, 961, 64, 1,
             None) == E_SHAPE                                                    # A+Nc > N
    assert c(P, P, P, P, P, P, 1088, P, 200, P, P, P, 1, 2, 2, 1088, 200, 1089, 64, 1,
             None) == E_SHAPE                                                    # Nc > N
    assert c(P, P, P, P, P, P, 900, None, 0, None, None, P, 1, 2, 2, 1088, 128, 960, 64, 1,
             None) == E_SHAPE                                                    # ldc < Nc
    assert c(P, P, P, P, P, P, 1088, P, 100, P, P, P, 1, 2, 2, 1088, 200, 1088, 64, 1,
             None) == E_SHAPE                                                    # ld_act < A
    assert c(P, P, P, P, P, P, 960, None, 0, None, None, P, 1, 2, 2, 1088, 64, 960, 64, 1,
             None) == E_UNSUP                                                    # one wave
    assert c(P, P, P, P, P, P, 960, None, 0, None, None, P, 3, 2, 2, 1088, 128, 960, 64, 1,
             None) == E_RANGE                                                    # no such mode
    assert c(P, P, P, P, P, P, 960, None, 0, None, None, BAD, 2, 2, 2, 1088, 128, 960, 64, 1,
             None) == E_RANGE


def test_status_strings(lib):
    for code in (OK, E_NULL, E_SHAPE, E_DTYPE, E_RANGE, E_WS, E_LAUNCH, E_UNSUP):
        s = lib.mar_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.mar_status_string(-99).decode() == "unknown status"
    assert lib.mar_version() >= 100


def attn(lib, q=P, ka=P, va=P, kc=P, vc=P, cidx=P, ldc=272, out=P, lse=None, B=2, H=2, N=320,
         A=48, Nc=272, D=64, scale=0.125, dtype=1):
    return lib.mar_cache_attn_fwd(q, ka, va, kc, vc, cidx, ldc, out, lse, B, H, N, A, Nc, D,
                                  scale, dtype, None)


def test_cache_attn_rejections(lib):
    assert attn(lib, q=None) == E_NULL
    assert attn(lib, out=None) == E_NULL
    assert attn(lib, cidx=None) == E_NULL          # Nc > 0 needs a list
    assert attn(lib, dtype=7) == E_DTYPE
    assert attn(lib, A=0) == E_SHAPE
    assert attn(lib, B=0) == E_SHAPE
    assert attn(lib, Nc=-1) == E_SHAPE
    assert attn(lib, A=49) == E_SHAPE              # A + Nc > N
    assert attn(lib, ldc=100) == E_SHAPE           # ldc < Nc
    assert attn(lib, D=128) == E_UNSUP
    assert attn(lib, scale=float("nan")) == E_RANGE
    assert attn(lib, scale=0.0) == E_RANGE
    assert attn(lib, scale=-0.125) == E_RANGE
    assert attn(lib, scale=float("inf")) == E_RANGE
    assert attn(lib, kc=BAD) == E_RANGE            # misaligned


def attn_upd(lib, q=P, ka=P, va=P, kc=P, vc=P, cidx=P, ldc=272, aidx=P, ld_act=48, err=None,
             out=P, lse=None, B=2, H=2, N=320, A=48, Nc=272, D=64, scale=0.125, dtype=1):
    return lib.mar_cache_attn_fwd_update(q, ka, va, kc, vc, cidx, ldc, aidx, ld_act, err, out, lse,
                                         B, H, N, A, Nc, D, scale, dtype, None)


def test_cache_attn_update_rejections(lib):
    assert attn_upd(lib, aidx=None) == E_NULL       # the active list is required ...
    assert attn_upd(lib, aidx=None, cidx=None, ldc=0, A=300, Nc=0) == E_NULL  # ... unless A == N
    assert attn_upd(lib, ld_act=47) == E_SHAPE      # ld_act < A
    assert attn_upd(lib, q=None) == E_NULL          # the attention's own checks apply
    assert attn_upd(lib, cidx=None) == E_NULL
    assert attn_upd(lib, A=49) == E_SHAPE
    assert attn_upd(lib, D=128) == E_UNSUP
    assert attn_upd(lib, scale=-1.0) == E_RANGE
    assert attn_upd(lib, kc=BAD) == E_RANGE
    assert attn_upd(lib, dtype=3) == E_DTYPE


def test_cache_attn_ragged_rejections(lib):
    f = lambda **kw: lib.mar_cache_attn_fwd_ragged(
        kw.get("q", P), P, P, P, P, kw.get("cidx", P), kw.get("ldc", 272), kw.get("al", P),
        kw.get("cl", P), P, None, 2, 2, 320, kw.get("A", 48), 272, 64, 0.125, 1, None)
    assert f(al=None) == E_NULL and f(cl=None) == E_NULL
    assert f(q=None) == E_NULL
    assert f(A=321) == E_SHAPE     # a capacity larger than N
    assert f(ldc=100) == E_SHAPE


def test_scatter_rejections(lib):
    f = lib.mar_kv_scatter_refresh
    assert f(None, P, P, P, P, 48, None, 2, 2, 320, 48, 64, 1, None) == E_NULL
    assert f(P, P, P, P, P, 48, None, 2, 2, 320, 48, 64, 9, None) == E_DTYPE
    assert f(P, P, P, P, None, 0, None, 2, 2, 320, 48, 64, 1, None) == E_SHAPE   # full needs M==N
    assert f(P, P, P, P, P, 10, None, 2, 2, 320, 48, 64, 1, None) == E_SHAPE     # ld_idx < M
    assert f(P, P, P, P, P, 48, None, 2, 2, 320, 48, 4, 1, None) == E_UNSUP      # 8-byte rows
    assert f(P, BAD, P, P, P, 48, None, 2, 2, 320, 48, 64, 1, None) == E_RANGE


def topk(lib, q=P, k=P, gp=P, ld_gp=256, n_gp=32, K=16, scores=P, act=P, ld_act=48, cac=P,
         ld_cac=272, clen=P, ws=P, ws_bytes=None, B=2, H=2, G=16, N=320, D=64, dtype=1):
    if ws_bytes is None:
        ws_bytes = B * H * N * 4
    return lib.mar_refresh_topk(q, k, gp, ld_gp, n_gp, K, 0.125, scores, act, ld_act, cac, ld_cac,
                                clen, ws, ws_bytes, B, H, G, N, D, dtype, None)


def test_topk_rejections(lib):
    assert lib.mar_refresh_topk_workspace(2, 3, 5) == 2 * 3 * 5 * 4
    assert lib.mar_refresh_topk_workspace(0, 3, 5) == 0
    assert topk(lib, scores=None) == E_NULL
    assert topk(lib, gp=None) == E_NULL
    assert topk(lib, dtype=3) == E_DTYPE
    assert topk(lib, K=-1) == E_RANGE
    assert topk(lib, K=300) == E_RANGE             # n_gp + K > N
    assert topk(lib, G=65) == E_UNSUP
    assert topk(lib, ld_act=40) == E_SHAPE
    assert topk(lib, ld_cac=100) == E_SHAPE
    assert topk(lib, ld_gp=10) == E_SHAPE
    assert topk(lib, N=5000, ld_cac=5000) == E_UNSUP
    assert topk(lib, ws=None) == E_WS
    assert topk(lib, ws_bytes=100) == E_WS


def test_layer2_scores_and_select_rejections(lib):
    f = lib.mar_cache_attn_fwd_scores
    # q, k, v, out, lse, gen, ld_gen, G, partials, bytes, B, H, N, D, scale, dtype, stream
    WS = 2 * 2 * 320 * 4
    assert f(None, P, P, P, None, P, 16, 16, P, WS, 2, 2, 320, 64, 0.125, 1, None) == E_NULL
    assert f(P, P, P, P, None, None, 16, 16, P, WS, 2, 2, 320, 64, 0.125, 1, None) == E_NULL
    assert f(P, P, P, P, None, P, 8, 16, P, WS, 2, 2, 320, 64, 0.125, 1, None) == E_SHAPE   # ld_gen < G
    assert f(P, P, P, P, None, P, 17, 17, P, WS, 2, 2, 320, 64, 0.125, 1, None) == E_UNSUP  # G > 16
    assert f(P, P, P, P, None, P, 16, 16, P, WS, 2, 2, 384, 64, 0.125, 1, None) == E_UNSUP  # N > 320
    assert f(P, P, P, P, None, P, 16, 16, P, WS, 2, 2, 64, 64, 0.125, 1, None) == E_UNSUP   # N <= 64
    assert f(P, P, P, P, None, P, 16, 16, P, WS, 2, 2, 320, 64, 0.125, 0, None) == E_UNSUP  # fp32
    assert f(P, P, P, P, None, P, 16, 16, P, WS - 4, 2, 2, 320, 64, 0.125, 1, None) == E_WS
    g = lib.mar_refresh_select
    # part, bytes, gp, ld_gp, n_gp, K, scores, act, ld_act, cached, ld_cached, len, B, H, G, N, s
    assert g(None, WS, P, 32, 32, 16, P, P, 48, P, 320, P, 2, 2, 16, 320, None) == E_NULL
    assert g(P, WS, P, 32, 32, 300, P, P, 332, P, 320, P, 2, 2, 16, 320, None) == E_RANGE
    assert g(P, WS, P, 32, 32, 16, P, P, 40, P, 320, P, 2, 2, 16, 320, None) == E_SHAPE    # ld_act
    assert g(P, WS - 4, P, 32, 32, 16, P, P, 48, P, 320, P, 2, 2, 16, 320, None) == E_WS
    assert g(P, WS, P, 32, 32, 16, P, P, 48, P, 320, P, 2, 2, 0, 320, None) == E_SHAPE     # G < 1


def test_refresh_topk_noalloc_rejections(lib):
    f = lib.mar_refresh_topk_noalloc
    # q, k, gp, ld_gp, n_gp, K, scale, scores, act, ld_act, cached, ld_cached, len, B, H, G, N, D, dt, s
    assert f(None, P, P, 4, 4, 4, 0.125, P, P, 8, P, 320, P, 2, 2, 4, 320, 64, 1, None) == E_NULL
    assert f(P, P, P, 4, 4, 400, 0.125, P, P, 404, P, 320, P, 2, 2, 4, 320, 64, 1, None) == E_RANGE
    assert f(P, P, P, 4, 4, 4, 0.125, P, P, 8, P, 320, P, 2, 2, 4, 320, 32, 1, None) == E_UNSUP
    # B*H*N floats beyond the library's 8 MiB array: refused before any GPU work
    assert 1024 * 16 * 320 * 4 > _lib.MAR_REFRESH_TOPK_SCRATCH_BYTES
    assert f(P, P, P, 4, 4, 4, 0.125, P, P, 8, P, 320, P, 1024, 16, 4, 320, 64, 1, None) == E_WS


def test_ragged_update_rejections(lib):
    f = lib.mar_cache_attn_fwd_ragged_update
    # q k v kc vc cached ldc act ld_act a_len c_len err out lse B H N A Nc D scale dtype stream
    ok = (P, P, P, P, P, P, 8, P, 32, P, P, None, P, None, 2, 2, 64, 32, 8, 64, 0.125, 1, None)
    assert f(*ok[:7], None, *ok[8:]) == E_NULL                          # no active list
    assert f(*ok[:9], None, *ok[10:]) == E_NULL                         # no a_len
    assert f(*ok[:10], None, *ok[11:]) == E_NULL                        # no c_len
    assert f(*ok[:8], 31, *ok[9:]) == E_SHAPE                           # ld_act < A
    assert f(*ok[:21], 0, None) == E_UNSUP                              # fp32
    assert f(*ok[:8], 8, *ok[9:17], 8, *ok[18:]) == E_UNSUP             # A < 16
    assert f(*ok[:17], 65, *ok[18:]) == E_SHAPE                         # capacity above N


def test_gate_and_cfg_rejections(lib):
    g = lib.mar_cos_gate
    assert g(None, P, 0.95, 1e-8, P, P, P, P, None, None, 2, 10, 64, 1, None) == E_NULL
    assert g(P, P, 0.95, 1e-8, P, P, P, P, P, None, 2, 10, 64, 1, None) == E_NULL  # one of the pair
    assert g(P, P, 0.95, 1e-8, P, P, P, P, None, P, 2, 10, 64, 1, None) == E_NULL
    assert g(P, P, 0.95, 1e-8, P, P, P, P, None, None, 2, 10, 64, 5, None) == E_DTYPE
    assert g(P, P, 0.95, 1e-8, P, P, P, P, P, P, 2, 0, 64, 1, None) == E_SHAPE
    assert g(P, P, 0.95, 1e-8, P, P, P, P, None, None, 2, 10, 12, 1, None) == E_UNSUP  # 24-byte rows
    assert g(P, P, float("nan"), 1e-8, P, P, P, P, None, None, 2, 10, 64, 1, None) == E_RANGE
    assert g(P, P, 0.95, -1.0, P, P, P, P, None, None, 2, 10, 64, 1, None) == E_RANGE
    c = lib.mar_cfg_residual
    assert c(P, P, P, None, None, 1.0, 5, 16, None) == E_RANGE                   # bad mode
    assert c(P, None, P, None, None, 1.0, 0, 16, None) == E_NULL                 # store needs uncond
    assert c(P, None, P, None, None, 1.0, 1, 16, None) == E_NULL                 # reuse needs out
    assert c(P, P, P, None, None, 1.0, 0, -1, None) == E_SHAPE
    assert c(P, BAD, P, None, None, 1.0, 0, 16, None) == E_RANGE


@pytest.mark.parametrize("name", ["mar_b", "mar_l", "mar_h", "highres"])
def test_plan_step_matches_oracle(lib, name):
    cfg = CONFIGS[name]
    counts = cosine_counts(cfg.n_img, cfg.steps)
    for warmup in (0, 2):
        for t in range(cfg.steps):
            ref = S.plan_step(counts, t, cfg.N, cfg.budget, 3, warmup)
            got = _lib.mar_plan_step(counts, t, cfg.N, cfg.budget, 3, warmup)
            assert got.refresh == int(ref.refresh)
            for f in ("step", "gen_begin", "n_gen", "prev_begin", "n_prev", "n_refresh",
                      "n_active", "n_cached"):
                assert getattr(got, f) == getattr(ref, f), (t, f)
            for layer in range(1, cfg.layers + 1):
                fl = _lib.mar_layer_flags(got, layer)
                assert bool(fl & _lib.MAR_LAYER_CACHE) == (S.layer_kind(ref, layer) == S.CACHE)
                assert bool(fl & _lib.MAR_LAYER_SELECT) == S.selects_refresh(ref, layer)
                assert bool(fl & _lib.MAR_LAYER_GATE) == S.gate_applies(ref, layer)


def test_plan_step_budget_clamp_golden(lib, golden_dir):
    """The library's planner on the hand-computed plans, including budgets that
    exceed the tokens outside G and P (K clamped to the eligible tokens)."""
    import json
    with open(os.path.join(golden_dir, "schedule_budget_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = _lib.mar_plan_step(c["counts"], c["step"], c["n_tokens"], c["budget"], c["period"])
        for k, v in c["plan"].items():
            assert int(getattr(got, k)) == v, (c["why"], k)


def test_plan_step_rejections(lib):
    plan = _lib.StepPlan()
    arr = (ctypes.c_int32 * 3)(1, 2, 3)
    p = ctypes.cast(arr, ctypes.c_void_p)
    assert lib.mar_plan_step(None, 3, 0, 10, 4, 3, 0, ctypes.byref(plan)) == E_NULL
    assert lib.mar_plan_step(p, 3, 3, 10, 4, 3, 0, ctypes.byref(plan)) == E_RANGE
    assert lib.mar_plan_step(p, 3, 0, 10, 4, 0, 0, ctypes.byref(plan)) == E_SHAPE
    assert lib.mar_plan_step(p, 3, 2, 5, 4, 3, 0, ctypes.byref(plan)) == E_RANGE  # 6 > 5 tokens
    assert lib.mar_layer_flags(None, 1, 2, 2, 3) == E_NULL
    with pytest.raises(_lib.MarError):
        _lib.mar_plan_step([1, 2], 5, 10, 4)
