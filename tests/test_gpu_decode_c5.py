"""The high-res (C5) decode through the library: MARché's cache-aware attention
with top-K refresh and LazyMAR's token cache, over a whole 64-step schedule,
checked against the oracle at every step.

Scaled to 1 image x 2 CFG sequences and 2 heads, at the high-res token count
(64 prefix + 1024 image tokens), an active budget of 128 and the cosine masking
schedule over 64 steps.  Three modelled layers per step:

* layer 2 (full attention) picks the refreshing tokens: top-K on the GPU's
  scores, bit-exact against the oracle's selection on those scores;
* layer 3 (MARché): the fused cache-aware attention + cache update of the
  active rows; on refresh steps (t % 3 == 0) full attention with the whole
  cache rewritten in the same call;
* layer 4 (LazyMAR token cache): the cosine gate picks each sequence's tokens
  to recompute; the ragged cache-aware attention runs those queries over
  their fresh K/V and the cached K/V of the reused tokens; the layer's cache
  then takes the recomputed rows (scatter with -1-padded lists).  On refresh
  steps every token is recomputed.

Fresh Q/K/V and gate features are redrawn every step, so the caches are stale
between refreshes exactly as in decoding.
"""
import numpy as np
import pytest
import torch

from mar_workloads import Config, cosine_counts, device_normal, gate_features, generation_order
from oracle import schedule as osched

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


@pytest.fixture(scope="module")
def marca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_attention_amd as m
    return m


def raw(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy()


def f64(t):
    return t.detach().double().cpu().numpy()


def gather_rows(x, idx):
    """x [B,H,N,D], idx [B,M] (non-negative) -> [B,H,M,D] (test-side indexing)."""
    B, H, N, D = x.shape
    i = idx.long()[:, None, :, None].expand(B, H, idx.shape[1], D)
    return torch.gather(x, 2, i).contiguous()


def check_unit(oracle, q, ka, va, kc, vc, cached, b, h, an, cn, got, what):
    sl = lambda t, n: f64(t[b:b + 1, h:h + 1, :n])
    cl = cached[b:b + 1, :max(cn, 1)]
    o, _ = oracle.cache_attention(sl(q, an), sl(ka, an), sl(va, an), f64(kc[b:b + 1, h:h + 1]),
                                  f64(vc[b:b + 1, h:h + 1]), cl, 0.125, Nc=cn)
    err = np.abs(f64(got[b, h, :an]) - o[0, 0]).max()
    assert err <= 2e-2, f"{what}: unit ({b},{h}) max-abs {err}"


def test_64_step_schedule_c5_token_cache(marca):
    import oracle
    cfg = Config("c5", B=2, H=2, D=64, N=1088, n_prefix=64, A=128, n_gen=0, n_prev=0, K=0,
                 layers=4, dtype="bf16", stale=True, budget=128, W=256, seed=4242)
    B, H, N, D = cfg.B, cfg.H, cfg.N, cfg.D
    bf = torch.bfloat16
    counts = cosine_counts(cfg.n_img, cfg.steps)
    assert counts.sum() == cfg.n_img
    order = torch.from_numpy(generation_order(cfg)).to(DEV)
    kc3, vc3, kc4, vc4 = (device_normal((B, H, N, D), 10 + i, DEV, bf) for i in range(4))
    n_refresh = 0
    for t in range(cfg.steps):
        plan = marca.mar_plan_step(counts, t, N, cfg.budget)
        ref = osched.plan_step(counts, t, N, cfg.budget)
        assert (bool(plan.refresh), plan.n_gen, plan.n_prev, plan.n_refresh, plan.n_active,
                plan.n_cached) == (ref.refresh, ref.n_gen, ref.n_prev, ref.n_refresh,
                                   ref.n_active, ref.n_cached), f"step {t}"
        seed = 5000 + 10 * t
        q2, k2, q3, k3, v3, q4, k4, v4 = (device_normal((B, H, N, D), seed + i, DEV, bf)
                                          for i in range(8))
        if plan.refresh:
            n_refresh += 1
            out3 = marca.mar_cache_attn_fwd_update(q3, k3, v3, kc3, vc3, None, None, Nc=0)
            out4 = marca.mar_cache_attn_fwd_update(q4, k4, v4, kc4, vc4, None, None, Nc=0)
            torch.cuda.synchronize()
            assert torch.equal(kc3, k3) and torch.equal(vc3, v3), f"step {t}: layer-3 refresh"
            assert torch.equal(kc4, k4) and torch.equal(vc4, v4), f"step {t}: layer-4 refresh"
            none = np.zeros((B, 1), np.int32)
            check_unit(oracle, q4, k4, v4, k4, v4, none, B - 1, 1, N, 0, out4, f"step {t} L4")
            continue

        # layer 2: the refresh selection from the generating queries' attention
        gp = order[:, plan.prev_begin:plan.gen_begin + plan.n_gen]
        gen_pos = order[:, plan.gen_begin:plan.gen_begin + plan.n_gen]
        q_gen = gather_rows(q2, gen_pos)
        scores, act, cac, clen = marca.mar_refresh_topk(q_gen, k2, gp, plan.n_prev + plan.n_gen,
                                                        plan.n_refresh)
        torch.cuda.synchronize()
        ra, rc, rl = oracle.refresh_select(f64(scores), gp.cpu().numpy(), plan.n_refresh,
                                           ld_cached=cac.shape[1])
        assert (act.cpu().numpy() == ra).all() and (cac.cpu().numpy() == rc).all(), f"step {t}"
        assert (clen.cpu().numpy() == plan.n_cached).all()

        # layer 3: cache-aware attention fused with the update of the active rows
        A, Nc = plan.n_active, plan.n_cached
        q_a, k_a, v_a = gather_rows(q3, act), gather_rows(k3, act), gather_rows(v3, act)
        kc3_0, vc3_0 = raw(kc3), raw(vc3)
        kc3_f, vc3_f = kc3.clone(), vc3.clone()
        out3 = marca.mar_cache_attn_fwd_update(q_a, k_a, v_a, kc3, vc3, cac, act, Nc=Nc)
        torch.cuda.synchronize()
        c_np = cac.cpu().numpy()
        check_unit(oracle, q_a, k_a, v_a, kc3_f, vc3_f, c_np, 0, 1, A, Nc, out3, f"step {t} L3")
        kr, vr, skipped = oracle.kv_scatter(kc3_0, vc3_0, raw(k_a), raw(v_a), act.cpu().numpy())
        assert skipped == 0
        assert np.array_equal(raw(kc3), kr) and np.array_equal(raw(vc3), vr), f"step {t}: L3 cache"

        # layer 4: the token gate, then the ragged attention over the recomputed
        # tokens and the cached K/V of the reused ones, then the cache update
        assert marca.mar_layer_flags(plan, 4) & marca.MAR_LAYER_GATE
        xg, yg, _ = gate_features(B, N, cfg.W, seed=seed + 9, device=DEV)
        cos, reuse, cidx, glen = marca.mar_cos_gate(xg, yg, cfg.tau)
        torch.cuda.synchronize()
        r2, c2, l2 = oracle.gate_from_cos(f64(cos), np.float32(cfg.tau))
        assert (reuse.cpu().numpy() == r2).all() and (cidx.cpu().numpy() == c2).all()
        n_comp = glen.cpu().numpy()
        A4 = int(n_comp.max())
        assert 0 < A4 < N
        comp = cidx[:, :A4].contiguous()
        q_c, k_c, v_c = (gather_rows(x, comp.clamp(min=0)) for x in (q4, k4, v4))
        reuse_pos = [torch.nonzero(reuse[b]).flatten().to(torch.int32) for b in range(B)]
        Nc4 = max(len(r) for r in reuse_pos)
        cached4 = torch.full((B, Nc4), -1, dtype=torch.int32, device=DEV)
        for b in range(B):
            cached4[b, :len(reuse_pos[b])] = reuse_pos[b]
        c_len4 = torch.tensor([len(r) for r in reuse_pos], dtype=torch.int32, device=DEV)
        assert ((c_len4 + glen) == N).all()
        out4 = marca.mar_cache_attn_fwd_ragged(q_c, k_c, v_c, kc4, vc4, cached4, glen, c_len4)
        torch.cuda.synchronize()
        c4_np = cached4.cpu().numpy()
        for b in range(B):
            check_unit(oracle, q_c, k_c, v_c, kc4, vc4, c4_np, b, b % H, int(n_comp[b]),
                       int(c_len4[b]), out4, f"step {t} L4")
        kc4_0, vc4_0 = raw(kc4), raw(vc4)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        marca.mar_kv_scatter_refresh(kc4, vc4, k_c, v_c, comp, err_count=err)
        torch.cuda.synchronize()
        kr, vr, skipped = oracle.kv_scatter(kc4_0, vc4_0, raw(k_c), raw(v_c), comp.cpu().numpy())
        assert skipped == int(err.item()) == int((comp < 0).sum())  # the -1 padding
        assert np.array_equal(raw(kc4), kr) and np.array_equal(raw(vc4), vr), f"step {t}: L4 cache"
    assert n_refresh == 22
