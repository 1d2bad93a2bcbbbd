"""The condition cache's half-batch steps (LazyMAR condition cache): between
refreshes only the conditional branch of each image's CFG pair is computed,
and the unconditional output is taken from the stored residual.  With the
conditional sequences first in the batch, that step is the same entry points
called on the first B/2 sequences (views of the same memory).

Every result of a sequence depends only on that sequence's inputs, and at the
MAR-L shape both batch sizes run the same per-unit code (one wave per unit:
1,024 and 2,048 units), so the half-batch calls must reproduce the first half
of the full-batch results bit for bit: attention, the fused cache update, the
full-attention layers, the refresh top-K and the token gate.  Two units of
the half batch are also checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

from mar_workloads import (CONFIGS, attention_inputs, device_gate_features, device_normal,
                           generation_order)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


@pytest.fixture(scope="module")
def marca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_attention_amd as m
    return m


def f64(t):
    return t.detach().double().cpu().numpy()


def test_conditional_half_attention_and_update(marca):
    import oracle
    cfg = CONFIGS["mar_l"]
    nb = cfg.B_img
    x = attention_inputs(cfg, DEV, seed=5150)
    qa, ka, va, kc, vc = (x[k] for k in ("q_a", "k_a", "v_a", "k_cache", "v_cache"))
    cached, active = x["cached"], x["active"]
    full = marca.mar_cache_attn_fwd(qa, ka, va, kc, vc, cached, Nc=cfg.Nc)
    half = marca.mar_cache_attn_fwd(qa[:nb], ka[:nb], va[:nb], kc[:nb], vc[:nb], cached[:nb],
                                    Nc=cfg.Nc)
    torch.cuda.synchronize()
    assert torch.equal(half, full[:nb])
    cl = cached.cpu().numpy()
    for b, h in [(0, 0), (nb - 1, cfg.H - 1)]:
        sl = lambda t: f64(t[b:b + 1, h:h + 1])
        o, _ = oracle.cache_attention(sl(qa), sl(ka), sl(va), sl(kc), sl(vc), cl[b:b + 1],
                                      cfg.D ** -0.5, Nc=cfg.Nc)
        assert np.abs(f64(half[b, h]) - o[0, 0]).max() <= 2e-2, (b, h)

    # the fused update on the half batch writes the conditional caches only
    kc2, vc2 = kc.clone(), vc.clone()
    kc3, vc3 = kc.clone(), vc.clone()
    outf = marca.mar_cache_attn_fwd_update(qa, ka, va, kc2, vc2, cached, active, Nc=cfg.Nc)
    outh = marca.mar_cache_attn_fwd_update(qa[:nb], ka[:nb], va[:nb], kc3[:nb], vc3[:nb],
                                           cached[:nb], active[:nb], Nc=cfg.Nc)
    torch.cuda.synchronize()
    assert torch.equal(outh, outf[:nb]) and torch.equal(outh, half)
    assert torch.equal(kc3[:nb], kc2[:nb]) and torch.equal(vc3[:nb], vc2[:nb])
    assert torch.equal(kc3[nb:], kc[nb:]) and torch.equal(vc3[nb:], vc[nb:])


def test_conditional_half_full_attention(marca):
    cfg = CONFIGS["mar_l"]
    nb = cfg.B_img
    q, k, v = (device_normal((cfg.B, cfg.H, cfg.N, cfg.D), 61 + i, DEV, torch.bfloat16)
               for i in range(3))
    full = marca.mar_cache_attn_fwd(q, k, v, k, v, None, Nc=0)
    half = marca.mar_cache_attn_fwd(q[:nb], k[:nb], v[:nb], k[:nb], v[:nb], None, Nc=0)
    torch.cuda.synchronize()
    assert torch.equal(half, full[:nb])


def test_conditional_half_topk_and_gate(marca):
    cfg = CONFIGS["mar_l"]
    nb = cfg.B_img
    order = torch.from_numpy(generation_order(cfg)).to(DEV)
    gp = order[:, 96:128]
    q = device_normal((cfg.B, cfg.H, cfg.n_gen, cfg.D), 71, DEV, torch.bfloat16)
    k = device_normal((cfg.B, cfg.H, cfg.N, cfg.D), 72, DEV, torch.bfloat16)
    full = marca.mar_refresh_topk(q, k, gp, 32, cfg.K)
    half = marca.mar_refresh_topk(q[:nb], k[:nb], gp[:nb], 32, cfg.K)
    torch.cuda.synchronize()
    for a, b in zip(half, full):
        assert torch.equal(a, b[:nb])

    gx, gy, _ = device_gate_features(cfg.B, cfg.N, cfg.W, seed=9, device=DEV)
    full = marca.mar_cos_gate(gx, gy, 0.95)
    half = marca.mar_cos_gate(gx[:nb], gy[:nb], 0.95)
    torch.cuda.synchronize()
    for a, b in zip(half, full):
        assert torch.equal(a, b[:nb])
