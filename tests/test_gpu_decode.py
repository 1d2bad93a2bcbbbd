"""A whole 64-step decode schedule through the library, checked against the oracle
at every step.

Scaled-down MAR-H-like shape (2 images x 2 CFG = 4 sequences, 2 heads, N = 64
prefix + 256 image tokens, active budget 64, cosine masking schedule over 64
steps), with two modelled layers per step: layer 2 (full attention, picks the
refreshing tokens) and layer 3 (cache-aware attention with its cache update).
Fresh Q/K/V are redrawn every step, so the cache is stale between refreshes
exactly as in decoding.  Per step:

* the host plan (mar_plan_step) against the oracle's schedule;
* refresh steps (t % 3 == 0): full attention of all N tokens and the full
  cache rewrite in one call, after which the cache equals the fresh K/V byte
  for byte; the CFG residual is stored;
* other steps: the top-K refresh selection from layer-2 scores (bit-exact on
  the GPU's scores; the partition covers every token once), the fused
  cache-aware attention + cache update (outputs against the oracle on the
  cache as it was; the cache afterwards against the oracle's scatter, byte
  for byte), the cosine gate on layer 4 when the layer roles say it applies,
  and the CFG reuse.
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
    """x [B,H,N,D], idx [B,M] -> [B,H,M,D] (test-side indexing)."""
    B, H, N, D = x.shape
    i = idx.long()[:, None, :, None].expand(B, H, idx.shape[1], D)
    return torch.gather(x, 2, i).contiguous()


def test_64_step_schedule(marca):
    import oracle
    cfg = Config("decode", B=4, H=2, D=64, N=320, n_prefix=64, A=64, n_gen=0, n_prev=0, K=0,
                 layers=4, dtype="bf16", stale=True, budget=64, W=256, seed=2024)
    B, H, N, D = cfg.B, cfg.H, cfg.N, cfg.D
    scale = D ** -0.5
    counts = cosine_counts(cfg.n_img, cfg.steps)
    assert counts.sum() == cfg.n_img and (counts >= 1).all()
    order = torch.from_numpy(generation_order(cfg)).to(DEV)
    bf = torch.bfloat16
    kc = device_normal((B, H, N, D), 1, DEV, bf)  # layer-3 caches (overwritten at step 0)
    vc = device_normal((B, H, N, D), 2, DEV, bf)
    c_prev, u_prev = None, None
    residual = None
    n_refresh_steps = 0
    for t in range(cfg.steps):
        plan = marca.mar_plan_step(counts, t, N, cfg.budget)
        ref = osched.plan_step(counts, t, N, cfg.budget)
        assert (bool(plan.refresh), plan.n_gen, plan.n_prev, plan.n_refresh, plan.n_active,
                plan.n_cached) == (ref.refresh, ref.n_gen, ref.n_prev, ref.n_refresh,
                                   ref.n_active, ref.n_cached), f"step {t}"
        seed = 1000 + 10 * t
        q2 = device_normal((B, H, N, D), seed + 1, DEV, bf)
        k2 = device_normal((B, H, N, D), seed + 2, DEV, bf)
        q3 = device_normal((B, H, N, D), seed + 3, DEV, bf)
        k3 = device_normal((B, H, N, D), seed + 4, DEV, bf)
        v3 = device_normal((B, H, N, D), seed + 5, DEV, bf)
        cond = torch.from_numpy(np.random.default_rng(seed).standard_normal((2, 64, 16))
                                .astype(np.float32)).to(DEV)
        uncond = cond - 0.1
        if plan.refresh:
            n_refresh_steps += 1
            # every layer full attention, and every cache row rewritten: layer 3
            # does both in one call (no active list); spot-check two units
            out = marca.mar_cache_attn_fwd_update(q3, k3, v3, kc, vc, None, None, Nc=0)
            torch.cuda.synchronize()
            for b, h in ((0, 0), (B - 1, H - 1)):
                sl = lambda x: f64(x[b:b + 1, h:h + 1])
                o, _ = oracle.cache_attention(sl(q3), sl(k3), sl(v3), sl(k3), sl(v3),
                                              np.zeros((1, 1), np.int32), scale, Nc=0)
                assert np.abs(f64(out[b, h]) - o[0, 0]).max() <= 2e-2, f"step {t}"
            assert torch.equal(kc, k3) and torch.equal(vc, v3), f"step {t}: full refresh"
            residual, _ = marca.mar_cfg_residual(cond, uncond)
            torch.cuda.synchronize()
            rr, _ = oracle.cfg_residual(cond.cpu().numpy(), uncond.cpu().numpy(), mode=0)
            assert (residual.cpu().numpy() == rr).all()
            continue

        # layer 2: refresh selection from the generating queries' attention
        n_gp = plan.n_prev + plan.n_gen
        gp = order[:, plan.prev_begin:plan.gen_begin + plan.n_gen]
        gen_pos = order[:, plan.gen_begin:plan.gen_begin + plan.n_gen]
        q_gen = gather_rows(q2, gen_pos)
        scores, act, cac, clen = marca.mar_refresh_topk(q_gen, k2, gp, n_gp, plan.n_refresh)
        torch.cuda.synchronize()
        s_ref = oracle.refresh_scores(f64(q_gen), f64(k2), scale)
        s_gpu = f64(scores)
        assert np.abs(s_gpu - s_ref).max() / np.abs(s_ref).max() <= 1e-5, f"step {t}"
        ra, rc, rl = oracle.refresh_select(s_gpu, gp.cpu().numpy(), plan.n_refresh,
                                           ld_cached=cac.shape[1])
        assert (act.cpu().numpy() == ra).all() and (cac.cpu().numpy() == rc).all(), f"step {t}"
        assert (clen.cpu().numpy() == plan.n_cached).all()
        a_np, c_np = act.cpu().numpy(), cac.cpu().numpy()
        for b in range(B):
            allv = np.concatenate([a_np[b], c_np[b, :plan.n_cached]])
            assert sorted(allv.tolist()) == list(range(N)), f"step {t}: partition"

        # layer 3: cache-aware attention fused with the cache update
        A, Nc = plan.n_active, plan.n_cached
        q_a, k_a, v_a = gather_rows(q3, act), gather_rows(k3, act), gather_rows(v3, act)
        kc0, vc0 = raw(kc), raw(vc)
        kc_before, vc_before = f64(kc), f64(vc)
        out = marca.mar_cache_attn_fwd_update(q_a, k_a, v_a, kc, vc, cac, act, Nc=Nc)
        torch.cuda.synchronize()
        for b, h in ((0, 1), (B - 1, 0), (1, 1)):
            sl = lambda x: f64(x[b:b + 1, h:h + 1])
            o, _ = oracle.cache_attention(sl(q_a), sl(k_a), sl(v_a),
                                          kc_before[b:b + 1, h:h + 1],
                                          vc_before[b:b + 1, h:h + 1],
                                          c_np[b:b + 1, :Nc], scale, Nc=Nc)
            assert np.abs(f64(out[b, h]) - o[0, 0]).max() <= 2e-2, f"step {t} unit {b},{h}"
        kr, vr, skipped = oracle.kv_scatter(kc0, vc0, raw(k_a), raw(v_a), a_np)
        assert skipped == 0
        assert np.array_equal(raw(kc), kr) and np.array_equal(raw(vc), vr), f"step {t}: cache"

        # layer 4: the token gate applies on reuse steps past the ungated layers
        flags = marca.mar_layer_flags(plan, 4)
        assert flags & marca.MAR_LAYER_GATE
        xg, yg, _ = gate_features(B, N, cfg.W, seed=seed + 7, device=DEV)
        cos, reuse, cidx, glen = marca.mar_cos_gate(xg, yg, 0.95)
        torch.cuda.synchronize()
        r2, c2, l2 = oracle.gate_from_cos(f64(cos), np.float32(0.95))
        assert (reuse.cpu().numpy() == r2).all() and (cidx.cpu().numpy() == c2).all()
        assert (glen.cpu().numpy() == l2).all()

        # CFG: the unconditional output comes from the stored residual
        u2, _ = marca.mar_cfg_residual(cond, residual=residual, mode=marca.MAR_CFG_REUSE)
        torch.cuda.synchronize()
        ur, _ = oracle.cfg_residual(cond.cpu().numpy(), residual=residual.cpu().numpy(), mode=1)
        assert (u2.cpu().numpy() == ur).all()
    assert n_refresh_steps == 22
