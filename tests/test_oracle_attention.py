"""Pins of the oracle's cache-aware attention against what the pages and the
mathematics fix (no GPU).

The method pages state that splitting attention into an active path and a
cached path and merging them with the safe online softmax is exactly standard
bidirectional softmax attention whenever the cache is current ("MARche"
paper-notes page, Key Design 2, Eq. 1-2; Pith review page, "What carries the
argument").  Each test below would fail for a plausible mistake in the oracle:
a dropped path, a wrong gather index, a missing normalisation, a wrong scale,
a transposed operand or an unstable exponent.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from mar_workloads import normal


def sdpa(q, k, v, scale):
    """Library softmax attention (torch, float64, CPU) of q [.., A, D] over k, v [.., N, D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q))
    kt = torch.from_numpy(np.ascontiguousarray(k))
    vt = torch.from_numpy(np.ascontiguousarray(v))
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale).numpy()


def split_inputs(q_full, k_full, v_full, active, cached):
    """Gather fresh active rows; the cache holds every fresh row."""
    q_a = q_full[:, :, active, :]
    k_a = k_full[:, :, active, :]
    v_a = v_full[:, :, active, :]
    return q_a, k_a, v_a


def test_current_cache_equals_full_attention():
    rng = np.random.default_rng(5)
    B, H, N, D = 2, 3, 40, 16
    q = normal((B, H, N, D), 1, 1)
    k = normal((B, H, N, D), 1, 2)
    v = normal((B, H, N, D), 1, 3)
    active = np.sort(rng.choice(N, 7, replace=False))
    cached = np.setdiff1d(np.arange(N), active)
    q_a, k_a, v_a = split_inputs(q, k, v, active, cached)
    idx = np.tile(cached.astype(np.int32), (B, 1))
    out, lse = oracle.cache_attention(q_a, k_a, v_a, k, v, idx, 0.25)
    ref = sdpa(q_a, k, v, 0.25)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    ref_lse = scipy.special.logsumexp(0.25 * np.einsum("bhad,bhnd->bhan", q_a, k), axis=-1)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_every_partition_of_a_tiny_sequence():
    """All 2^N - 1 non-empty active sets of N = 8 tokens give full attention."""
    N, D = 8, 4
    q = normal((1, 1, N, D), 2, 1)
    k = normal((1, 1, N, D), 2, 2)
    v = normal((1, 1, N, D), 2, 3)
    full = sdpa(q, k, v, 0.5)
    for r in range(1, N + 1):
        for act in itertools.combinations(range(N), r):
            active = np.array(act)
            cached = np.setdiff1d(np.arange(N), active).astype(np.int32)
            q_a, k_a, v_a = split_inputs(q, k, v, active, cached)
            idx = cached[None, :] if cached.size else np.zeros((1, 0), np.int32)
            out, _ = oracle.cache_attention(q_a, k_a, v_a, k, v, idx, 0.5, Nc=cached.size)
            np.testing.assert_allclose(out[0, 0], full[0, 0, active], rtol=1e-12, atol=1e-13)


def test_identity_values_return_softmax_rows():
    """With V = I the output rows are the attention probabilities themselves."""
    N = D = 64
    A = 8
    q = normal((1, 2, A, D), 3, 1)
    k = normal((1, 2, N, D), 3, 2)
    eye = np.broadcast_to(np.eye(N), (1, 2, N, D)).copy()
    active = np.arange(A) * 5
    cached = np.setdiff1d(np.arange(N), active).astype(np.int32)
    k_a = k[:, :, active]
    v_a = eye[:, :, active]
    out, _ = oracle.cache_attention(q, k_a, v_a, k, eye, cached[None], 0.125)
    # out[..., i, n] is the weight of token n (active tokens via v_a rows = e_active)
    logits = 0.125 * np.einsum("bhad,bhnd->bhan", q, k)
    np.testing.assert_allclose(out, scipy.special.softmax(logits, axis=-1), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert (out >= 0).all()


def test_closed_forms(golden_dir):
    with open(os.path.join(golden_dir, "attention_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], float)[None, None]
        ka = np.array(c["ka"], float)[None, None]
        va = np.array(c["va"], float)[None, None]
        kc = np.array(c["kc"], float)[None, None]
        vc = np.array(c["vc"], float)[None, None]
        # the cache holds only the cached rows here: positions 0..Nc-1
        Nc = kc.shape[2]
        idx = np.arange(Nc, dtype=np.int32)[None]
        out, lse = oracle.cache_attention(q, ka, va, kc, vc, idx, c["scale"])
        np.testing.assert_allclose(out[0, 0], np.array(c["out"]), rtol=0, atol=1e-12,
                                   err_msg=c["name"])
        np.testing.assert_allclose(lse[0, 0], np.array(c["lse"]), rtol=1e-14, atol=1e-12,
                                   err_msg=c["name"])


def test_constant_values_and_single_query():
    B, H, A, N, D = 1, 2, 1, 30, 8
    q = normal((B, H, A, D), 4, 1) * 3.0
    k = normal((B, H, N, D), 4, 2)
    v = np.full((B, H, N, D), -1.75)
    cached = np.arange(1, N, dtype=np.int32)[None]
    out, _ = oracle.cache_attention(q, k[:, :, :1], v[:, :, :1], k, v, cached, 0.3)
    np.testing.assert_allclose(out, -1.75, rtol=0, atol=1e-14)
    # A = 1: a single softmax row, compared with scipy's softmax
    v = normal((B, H, N, D), 4, 3)
    out, _ = oracle.cache_attention(q, k[:, :, :1], v[:, :, :1], k, v, cached, 0.3)
    p = scipy.special.softmax(0.3 * np.einsum("bhad,bhnd->bhan", q, k), axis=-1)
    np.testing.assert_allclose(out, np.einsum("bhan,bhnd->bhad", p, v), rtol=1e-12, atol=1e-14)


def test_cached_order_does_not_matter():
    B, H, A, N, D = 2, 2, 5, 50, 8
    rng = np.random.default_rng(9)
    q = normal((B, H, A, D), 5, 1)
    ka = normal((B, H, A, D), 5, 2)
    va = normal((B, H, A, D), 5, 3)
    kc = normal((B, H, N, D), 5, 4)
    vc = normal((B, H, N, D), 5, 5)
    idx = np.stack([rng.choice(N, 31, replace=False) for _ in range(B)]).astype(np.int32)
    out1, lse1 = oracle.cache_attention(q, ka, va, kc, vc, idx, 0.35)
    perm = np.stack([rng.permutation(idx[b]) for b in range(B)]).astype(np.int32)
    out2, lse2 = oracle.cache_attention(q, ka, va, kc, vc, perm, 0.35)
    np.testing.assert_allclose(out1, out2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-14)


def test_stale_cache_rows_are_the_defined_input():
    """With a stale cache the result is attention over [K_A ; stale K_C] (not fresh)."""
    B, H, N, D, A = 1, 2, 24, 8, 6
    q = normal((B, H, A, D), 6, 1)
    k = normal((B, H, N, D), 6, 2)
    v = normal((B, H, N, D), 6, 3)
    ks = k + 0.33 * normal((B, H, N, D), 6, 4)
    vs = v + 0.33 * normal((B, H, N, D), 6, 5)
    active = np.array([1, 4, 9, 10, 17, 23])
    cached = np.setdiff1d(np.arange(N), active).astype(np.int32)
    out, _ = oracle.cache_attention(q, k[:, :, active], v[:, :, active], ks, vs, cached[None], 0.2)
    kk = np.concatenate([k[:, :, active], ks[:, :, cached]], axis=2)
    vv = np.concatenate([v[:, :, active], vs[:, :, cached]], axis=2)
    np.testing.assert_allclose(out, sdpa(q, kk, vv, 0.2), rtol=1e-12, atol=1e-13)
    fresh = sdpa(q, k, v, 0.2)
    assert np.abs(out - fresh).max() > 1e-3


def test_lse_merges_the_two_paths():
    """lse over both paths = logaddexp of each path's own log-sum-exp."""
    B, H, A, N, D = 1, 1, 4, 20, 8
    q = normal((B, H, A, D), 7, 1)
    ka = normal((B, H, A, D), 7, 2)
    va = normal((B, H, A, D), 7, 3)
    kc = normal((B, H, N, D), 7, 4)
    vc = normal((B, H, N, D), 7, 5)
    idx = np.arange(3, 19, dtype=np.int32)[None]
    _, lse = oracle.cache_attention(q, ka, va, kc, vc, idx, 0.4)
    la = scipy.special.logsumexp(0.4 * np.einsum("bhad,bhnd->bhan", q, ka), axis=-1)
    lc = scipy.special.logsumexp(0.4 * np.einsum("bhad,bhnd->bhan", q, kc[:, :, 3:19]), axis=-1)
    np.testing.assert_allclose(lse, np.logaddexp(la, lc), rtol=1e-13)


def test_empty_cached_set_and_bad_index():
    B, H, A, D = 1, 1, 3, 4
    q = normal((B, H, A, D), 8, 1)
    ka = normal((B, H, A, D), 8, 2)
    va = normal((B, H, A, D), 8, 3)
    kc = np.zeros((B, H, 5, D))
    out, _ = oracle.cache_attention(q, ka, va, kc, kc, np.zeros((1, 0), np.int32), 1.0, Nc=0)
    np.testing.assert_allclose(out, sdpa(q, ka, va, 1.0), rtol=1e-12, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.cache_attention(q, ka, va, kc, kc, np.array([[5]], np.int32), 1.0)
