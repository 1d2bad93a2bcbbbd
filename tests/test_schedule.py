"""Pins of the oracle's step schedule and of the workload's masking schedule (no GPU)."""
import json
import os

import numpy as np

from mar_workloads import CONFIGS, cosine_counts, generation_order
from oracle import schedule as S


def test_refresh_steps_golden(golden_dir):
    with open(os.path.join(golden_dir, "schedule_refresh_steps.json")) as f:
        g = json.load(f)
    counts = cosine_counts(256, g["steps"])
    plans = [S.plan_step(counts, t, 320, 48, g["period"]) for t in range(g["steps"])]
    refresh = [p.step for p in plans if p.refresh]
    assert refresh == g["refresh_steps"]
    assert len(refresh) == g["n_refresh"]
    assert sum(not p.refresh for p in plans) == g["n_cache_aware"]


def test_budget_clamp_golden(golden_dir):
    """Hand-computed plans, including budgets larger than the tokens left once
    G and P are taken, where K is clamped to the eligible tokens."""
    with open(os.path.join(golden_dir, "schedule_budget_cases.json")) as f:
        cases = json.load(f)["cases"]
    assert sum(c["plan"]["n_refresh"] < c["budget"] - c["plan"]["n_gen"] - c["plan"]["n_prev"]
               for c in cases) >= 3  # the upper clamp binds in at least three cases
    for c in cases:
        p = S.plan_step(c["counts"], c["step"], c["n_tokens"], c["budget"], c["period"])
        for k, v in c["plan"].items():
            assert int(getattr(p, k)) == v, (c["why"], k)


def test_cosine_counts():
    for n_img, steps in [(256, 64), (1024, 64), (256, 16), (64, 64)]:
        c = cosine_counts(n_img, steps)
        assert c.sum() == n_img and (c >= 1).all() and c.size == steps
    c = cosine_counts(256, 64)
    assert c[0] == 1 and c.max() <= 8
    # the cosine schedule generates few tokens first and more later
    assert c[:8].sum() < c[-8:].sum()


def test_plan_budget_and_slices():
    counts = cosine_counts(256, 64)
    N, budget = 320, 64
    for t in range(64):
        p = S.plan_step(counts, t, N, budget)
        assert p.gen_begin == counts[:t].sum()
        assert p.n_gen == counts[t]
        if t > 0:
            assert p.prev_begin + p.n_prev == p.gen_begin  # P then G is one slice
        if p.refresh:
            assert p.n_active == N and p.n_cached == 0
        else:
            assert p.n_refresh == max(0, budget - p.n_gen - p.n_prev)
            assert p.n_active == p.n_gen + p.n_prev + p.n_refresh
            assert p.n_active + p.n_cached == N
    # a budget smaller than G + P gives K = 0
    p = S.plan_step([5, 5, 5], 1, 100, 4)
    assert p.n_refresh == 0 and p.n_active == 10


def test_layer_roles():
    counts = cosine_counts(256, 64)
    p_ref = S.plan_step(counts, 3, 320, 48)
    p_c = S.plan_step(counts, 4, 320, 48)
    assert p_ref.refresh and not p_c.refresh
    assert [S.layer_kind(p_ref, l) for l in (1, 2, 3, 32)] == [S.FULL] * 4
    assert [S.layer_kind(p_c, l) for l in (1, 2, 3, 32)] == [S.FULL, S.FULL, S.CACHE, S.CACHE]
    assert S.selects_refresh(p_c, 2) and not S.selects_refresh(p_c, 3)
    assert not S.selects_refresh(p_ref, 2)
    assert [S.gate_applies(p_c, l) for l in (1, 3, 4)] == [False, False, True]
    assert S.cfg_mode(p_ref) == "store" and S.cfg_mode(p_c) == "reuse"
    # warm-up steps are full
    assert S.plan_step(counts, 1, 320, 48, warmup=2).refresh


def test_generation_order_shared_by_cfg_pair():
    cfg = CONFIGS["mar_b"]
    order = generation_order(cfg)
    assert order.shape == (cfg.B, cfg.n_img)
    assert (order[:cfg.B_img] == order[cfg.B_img:]).all()
    for b in range(3):
        assert sorted(order[b].tolist()) == list(range(cfg.n_prefix, cfg.N))
