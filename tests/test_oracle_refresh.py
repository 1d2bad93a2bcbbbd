"""Pins of the oracle's refresh scores and top-K selection (no GPU).

Selection rule ("MARche" paper-notes page, Key Design 1; figure 3 caption on
the Pith review page): in layer 2, attention weights from every generating
token to every token are averaged over heads; the K tokens with the highest
scores refresh, alongside the generating and previous-step caching tokens.
"""
import itertools
import json
import os

import numpy as np
import scipy.special

import oracle
from mar_workloads import normal


def test_scores_sum_to_one_and_single_row_is_softmax():
    B, H, G, N, D = 3, 4, 5, 37, 16
    q = normal((B, H, G, D), 10, 1)
    k = normal((B, H, N, D), 10, 2)
    s = oracle.refresh_scores(q, k, 0.25)
    np.testing.assert_allclose(s.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert (s > 0).all()
    # H = G = 1: the scores are one softmax row
    s1 = oracle.refresh_scores(q[:, :1, :1], k[:, :1], 0.25)
    ref = scipy.special.softmax(0.25 * np.einsum("bd,bnd->bn", q[:, 0, 0], k[:, 0]), axis=-1)
    np.testing.assert_allclose(s1, ref, rtol=1e-12, atol=1e-16)


def test_scores_average_over_heads_and_queries():
    B, G, N, D = 2, 3, 20, 8
    q = normal((B, 1, G, D), 11, 1)
    k = normal((B, 1, N, D), 11, 2)
    base = oracle.refresh_scores(q, k, 0.5)
    # repeating a head, or a query, leaves a mean unchanged
    s2 = oracle.refresh_scores(np.concatenate([q, q], 1), np.concatenate([k, k], 1), 0.5)
    np.testing.assert_allclose(s2, base, rtol=1e-13)
    s3 = oracle.refresh_scores(np.concatenate([q, q], 2), k, 0.5)
    np.testing.assert_allclose(s3, base, rtol=1e-13)
    # mean of two different single-query rows
    r0 = oracle.refresh_scores(q[:, :, :1], k, 0.5)
    r1 = oracle.refresh_scores(q[:, :, 1:2], k, 0.5)
    s01 = oracle.refresh_scores(q[:, :, :2], k, 0.5)
    np.testing.assert_allclose(s01, 0.5 * (r0 + r1), rtol=1e-13)


def test_scores_uniform_at_zero_scale_and_permutation_equivariant():
    B, H, G, N, D = 1, 2, 2, 12, 4
    q = normal((B, H, G, D), 12, 1)
    k = normal((B, H, N, D), 12, 2)
    np.testing.assert_allclose(oracle.refresh_scores(q, k, 0.0), 1.0 / N, rtol=1e-14)
    perm = np.random.default_rng(3).permutation(N)
    s = oracle.refresh_scores(q, k, 0.7)
    sp = oracle.refresh_scores(q, k[:, :, perm], 0.7)
    np.testing.assert_allclose(sp, s[:, perm], rtol=1e-13)


def test_duplicate_keys_tie_and_lower_index_wins():
    B, H, G, N, D = 1, 2, 3, 10, 8
    q = normal((B, H, G, D), 13, 1) * 2
    k = normal((B, H, N, D), 13, 2)
    k[:, :, 7] = k[:, :, 3]  # identical keys => bit-identical scores
    s = oracle.refresh_scores(q, k, 1.0)
    assert s[0, 3] == s[0, 7]
    # make token 3/7 the clear best and ask for one refreshing token
    k[:, :, 3] = k[:, :, 7] = 4.0 * np.sign(q.sum(2))
    s = oracle.refresh_scores(q, k, 1.0)
    active, cached, clen = oracle.refresh_select(s, np.array([[0]], np.int32), 1)
    assert active.tolist() == [[0, 3]]
    assert 7 in cached[0, :clen[0]]


def test_select_golden(golden_dir):
    with open(os.path.join(golden_dir, "topk_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        s = np.array(c["scores"], float)[None]
        gp = np.array(c["gp"], np.int32)[None]
        active, cached, clen = oracle.refresh_select(s, gp, c["K"])
        assert active[0].tolist() == c["active"], c["name"]
        assert cached[0].tolist() == c["cached"], c["name"]
        assert int(clen[0]) == c["cached_len"], c["name"]


def test_select_matches_stable_argsort_and_partitions():
    rng = np.random.default_rng(14)
    B, N, K = 6, 57, 11
    s = rng.random((B, N))
    s[:, 10:14] = 0.5  # a tie band
    gp = np.stack([rng.choice(N, 9, replace=False) for _ in range(B)]).astype(np.int32)
    active, cached, clen = oracle.refresh_select(s, gp, K)
    for b in range(B):
        elig = np.setdiff1d(np.arange(N), gp[b])
        order = elig[np.argsort(-s[b, elig], kind="stable")]  # stable => lower index first
        assert active[b, :9].tolist() == gp[b].tolist()
        assert active[b, 9:].tolist() == order[:K].tolist()
        rest = np.setdiff1d(np.arange(N), active[b])
        assert clen[b] == rest.size
        assert cached[b, :clen[b]].tolist() == rest.tolist()  # ascending complement
        assert (cached[b, clen[b]:] == -1).all()
        union = np.concatenate([active[b], cached[b, :clen[b]]])
        assert sorted(union.tolist()) == list(range(N))


def test_select_brute_force_subsets():
    """With distinct scores the chosen set is the unique K-subset of largest sum."""
    rng = np.random.default_rng(15)
    N, K = 9, 3
    for trial in range(20):
        s = rng.random((1, N))
        gp = rng.choice(N, 2, replace=False).astype(np.int32)[None]
        active, _, _ = oracle.refresh_select(s, gp, K)
        elig = [j for j in range(N) if j not in gp[0]]
        best = max(itertools.combinations(elig, K), key=lambda c: sum(s[0, list(c)]))
        assert sorted(active[0, 2:].tolist()) == sorted(best)
        # and in descending score order
        assert list(s[0, active[0, 2:]]) == sorted(s[0, active[0, 2:]], reverse=True)
