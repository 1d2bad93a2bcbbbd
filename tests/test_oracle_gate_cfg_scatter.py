"""Pins of the oracle's cosine gate, CFG residual cache and KV scatter (no GPU).

Gate and condition cache: "LazyMAR" paper-notes page, Key designs.  KV update
and full refresh: "MARche" abstract (only tokens needing recomputation are
updated) and paper-notes page, Key Design 3 (full refresh every 3 steps).
"""
import json
import math
import os

import numpy as np
import scipy.spatial.distance

import oracle
from mar_workloads import gate_features, normal


def test_gate_golden(golden_dir):
    with open(os.path.join(golden_dir, "gate_cases.json")) as f:
        groups = json.load(f)["groups"]
    for g in groups:
        x = np.array(g["x"], float)[None]
        y = np.array(g["y"], float)[None]
        cos, reuse, cidx, clen = oracle.cos_gate(x, y, g["tau"])
        np.testing.assert_allclose(cos[0], g["cos"], rtol=0, atol=1e-15)
        assert reuse[0].tolist() == g["reuse"]
        assert cidx[0].tolist() == g["compute_idx"]
        assert int(clen[0]) == g["compute_len"]


def test_gate_invariants_and_scipy():
    B, N, W = 2, 30, 64
    x = normal((B, N, W), 20, 1)
    y = normal((B, N, W), 20, 2)
    cos, _, _, _ = oracle.cos_gate(x, y, 0.95)
    ref = np.array([[1.0 - scipy.spatial.distance.cosine(x[b, j], y[b, j]) for j in range(N)]
                    for b in range(B)])
    np.testing.assert_allclose(cos, ref, rtol=0, atol=1e-14)
    c_same, r_same, _, l_same = oracle.cos_gate(x, x, 0.95)
    np.testing.assert_allclose(c_same, 1.0, atol=1e-14)
    assert (r_same == 1).all() and (l_same == 0).all()
    c_neg, _, _, _ = oracle.cos_gate(x, -x, 0.95)
    np.testing.assert_allclose(c_neg, -1.0, atol=1e-14)
    c_sc, _, _, _ = oracle.cos_gate(x, 3.5 * x, 0.95)
    np.testing.assert_allclose(c_sc, 1.0, atol=1e-14)


def test_gate_constructed_cosine():
    """y = rho * e1 + sqrt(1 - rho^2) * e2 against x = e1 has cosine rho."""
    rhos = np.array([-0.3, 0.0, 0.5, 0.9499, 0.95, 0.9501, 0.99])
    W = 5
    x = np.zeros((1, rhos.size, W))
    x[..., 0] = 1.0
    y = np.zeros((1, rhos.size, W))
    y[0, :, 0] = rhos
    y[0, :, 1] = np.sqrt(1 - rhos ** 2)
    cos, reuse, cidx, clen = oracle.cos_gate(x, y, 0.95)
    np.testing.assert_allclose(cos[0], rhos, atol=1e-15)
    assert reuse[0].tolist() == [0, 0, 0, 0, 1, 1, 1]
    assert cidx[0].tolist() == [0, 1, 2, 3, -1, -1, -1] and clen[0] == 4


def test_gate_workload_generator_hits_target_cosines():
    x, y, rho = gate_features(2, 50, 1024, seed=3, dtype="bf16")
    cos, reuse, cidx, clen = oracle.cos_gate(x, y, 0.95)
    assert np.abs(cos - rho).max() < 2e-3
    assert (reuse == (rho > 0.95)).all()
    # compaction: ascending, -1 padded, consistent with reuse
    for b in range(2):
        comp = np.nonzero(reuse[b] == 0)[0]
        assert cidx[b, :clen[b]].tolist() == comp.tolist()
        assert (cidx[b, clen[b]:] == -1).all()


def test_gate_from_cos_matches_gate():
    x = normal((3, 40, 16), 21, 1)
    y = x + 0.4 * normal((3, 40, 16), 21, 2)
    cos, reuse, cidx, clen = oracle.cos_gate(x, y, 0.9)
    r2, c2, l2 = oracle.gate_from_cos(cos, 0.9)
    assert (r2 == reuse).all() and (c2 == cidx).all() and (l2 == clen).all()


def test_cfg_golden(golden_dir):
    with open(os.path.join(golden_dir, "cfg_cases.json")) as f:
        g = json.load(f)
    st, ru, w = g["store"], g["reuse"], g["w"]
    res, guided = oracle.cfg_residual(np.array(st["cond"]), np.array(st["uncond"]), mode=0, w=w)
    assert res.tolist() == st["residual"] and guided.tolist() == st["guided"]
    uo, guided = oracle.cfg_residual(np.array(ru["cond"]), residual=np.array(ru["residual"]),
                                     mode=1, w=w)
    assert uo.tolist() == ru["uncond"] and guided.tolist() == ru["guided"]


def test_cfg_float32_rounding_and_round_trip():
    rng = np.random.default_rng(22)
    c = rng.standard_normal(4096).astype(np.float32)
    u = (c - rng.standard_normal(4096) / 6).astype(np.float32)
    res, _ = oracle.cfg_residual(c, u, mode=0)
    # IEEE float32 subtraction is correctly rounded: numpy's float32 result is the pin
    assert (res == (c - u)).all()
    c2 = (c + rng.standard_normal(4096)).astype(np.float32)
    uo, _ = oracle.cfg_residual(c2, residual=res, mode=1)
    assert (uo == (c2 - res)).all()
    # round trip: if uncond_t == cond_t - r by construction, reuse reproduces it
    uo2, _ = oracle.cfg_residual(c, residual=res, mode=1)
    assert (uo2 == (c - res)).all()
    # guided within one rounding of the exact value
    _, gd = oracle.cfg_residual(c, u, mode=0, w=1.5)
    exact = u.astype(np.float64) + 1.5 * (c.astype(np.float64) - u.astype(np.float64))
    assert np.abs(gd - exact).max() <= np.abs(exact).max() * 2.0 ** -23


def test_scatter_partial_full_and_skips():
    rng = np.random.default_rng(24)
    B, H, N, M, D = 2, 3, 20, 5, 8
    kc = rng.standard_normal((B, H, N, D)).astype(np.float32)
    vc = rng.standard_normal((B, H, N, D)).astype(np.float32)
    kn = rng.standard_normal((B, H, M, D)).astype(np.float32)
    vn = rng.standard_normal((B, H, M, D)).astype(np.float32)
    idx = np.stack([rng.choice(N, M, replace=False) for _ in range(B)]).astype(np.int32)
    k2, v2, sk = oracle.kv_scatter(kc, vc, kn, vn, idx)
    assert sk == 0
    ref_k, ref_v = kc.copy(), vc.copy()
    for b in range(B):
        ref_k[b][:, idx[b]] = kn[b]
        ref_v[b][:, idx[b]] = vn[b]
    assert (k2 == ref_k).all() and (v2 == ref_v).all()
    # gather(scatter(x)) == x, untouched rows unchanged
    for b in range(B):
        assert (k2[b][:, idx[b]] == kn[b]).all()
        untouched = np.setdiff1d(np.arange(N), idx[b])
        assert (k2[b][:, untouched] == kc[b][:, untouched]).all()
    # full refresh
    kf = rng.standard_normal((B, H, N, D)).astype(np.float32)
    vf = rng.standard_normal((B, H, N, D)).astype(np.float32)
    k3, v3, _ = oracle.kv_scatter(kc, vc, kf, vf, None)
    assert (k3 == kf).all() and (v3 == vf).all()
    # out-of-range indices are skipped and counted once per (b, m)
    bad = idx.copy()
    bad[0, 1] = N
    bad[1, 4] = -3
    k4, _, sk = oracle.kv_scatter(kc, vc, kn, vn, bad)
    assert sk == 2
    assert (k4[0][:, idx[0, 1]] == kc[0][:, idx[0, 1]]).all()
    # bf16 bytes (uint16 view) are copied bit for bit
    kb = rng.integers(0, 2 ** 16, (B, H, N, D), dtype=np.uint16)
    nb = rng.integers(0, 2 ** 16, (B, H, M, D), dtype=np.uint16)
    k5, _, _ = oracle.kv_scatter(kb, kb, nb, nb, idx)
    assert (k5[0][:, idx[0]] == nb[0]).all()
