"""GPU parity of mar_cache_attn_fwd_update (attention fused with the cache
update of the active rows) against the oracle.

The attention output follows the same tolerances as mar_cache_attn_fwd (bf16:
max-abs 2e-2, lse 4.5e-3; fp32: normwise 1e-5) and is also required to equal
mar_cache_attn_fwd bit for bit, since the fused kernel runs the same
arithmetic.  The caches must equal the oracle's row scatter byte for byte.
"""
import numpy as np
import pytest
import torch

from mar_workloads import CONFIGS, Config, attention_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


@pytest.fixture(scope="module")
def marca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_attention_amd as m
    return m


def raw(t):
    """The bytes of a device tensor as a numpy integer array (bit-exact compare)."""
    t = t.detach().contiguous().cpu()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def check_case(marca, x, Nc, active, dtype, units=None):
    import oracle
    cfg = x["cfg"]
    B, H, A, D = x["q_a"].shape
    cached = x["cached"][:, :Nc].contiguous() if Nc > 0 else None
    # reference: the unfused attention and the oracle's scatter on copies
    kc0, vc0 = x["k_cache"].clone(), x["v_cache"].clone()
    lse_ref = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out_ref = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], kc0, vc0, cached, Nc=Nc,
                                       lse=lse_ref)
    kc_o, vc_o, skipped = oracle.kv_scatter(raw(x["k_cache"]), raw(x["v_cache"]), raw(x["k_a"]),
                                            raw(x["v_a"]), active.cpu().numpy())
    # fused
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    lse = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd_update(x["q_a"], x["k_a"], x["v_a"], kc, vc, cached, active,
                                          Nc=Nc, lse=lse, err_count=err)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
    assert np.array_equal(raw(kc), kc_o) and np.array_equal(raw(vc), vc_o)
    assert int(err.item()) == skipped
    # the output against the oracle on a few units (attention over the cache
    # as it was before the update: the update touches no cached row)
    units = units or [(0, 0), (B - 1, H - 1)]
    tol = 2e-2 if dtype == "bf16" else None
    for b, h in units:
        sl = lambda t: t[b:b + 1, h:h + 1].double().cpu().numpy()
        cl = x["cached"][b:b + 1, :max(Nc, 1)].cpu().numpy()
        o, l = oracle.cache_attention(sl(x["q_a"]), sl(x["k_a"]), sl(x["v_a"]),
                                      sl(x["k_cache"]), sl(x["v_cache"]), cl, D ** -0.5, Nc=Nc)
        got = out[b, h].double().cpu().numpy()
        if tol is not None:
            assert np.abs(got - o[0, 0]).max() <= tol
        else:
            assert np.abs(got - o[0, 0]).max() / np.abs(o[0, 0]).max() <= 1e-5
    return skipped


def small(dtype, B, H, N, A, seed):
    return Config("t", B=B, H=H, D=64, N=N, n_prefix=0, A=A, n_gen=0, n_prev=0, K=0, layers=1,
                  dtype=dtype, stale=True, seed=seed)


@pytest.mark.parametrize("dtype,A,Nc", [("bf16", 16, 48), ("bf16", 48, 272), ("bf16", 33, 1),
                                        ("bf16", 100, 37), ("bf16", 128, 160), ("bf16", 8, 50),
                                        ("f32", 24, 40), ("bf16", 64, 0),
                                        # the K rows are stored 8 whole rows at a time:
                                        # 21 active rows end inside such a group
                                        ("bf16", 21, 11)])
def test_fused_update_matches_attention_and_scatter(marca, dtype, A, Nc):
    cfg = small(dtype, 2, 3, A + Nc + 3, A, seed=900 + A + Nc)
    x = attention_inputs(cfg, DEV, ascending=False)
    active = x["active"].to(torch.int32).contiguous()
    assert check_case(marca, x, Nc, active, dtype) == 0


def test_fused_update_skips_and_counts_invalid_entries(marca):
    cfg = small("bf16", 2, 3, 330, 48, seed=77)
    x = attention_inputs(cfg, DEV, ascending=False)
    active = x["active"].to(torch.int32).clone()
    active[0, 5] = -1
    active[1, 40] = 330 + 2
    active = active.contiguous()
    assert check_case(marca, x, cfg.N - cfg.A, active, "bf16") == 2


def test_fused_update_full_size_mar_l(marca):
    cfg = CONFIGS["mar_l"]
    x = attention_inputs(cfg, DEV)
    active = x["active"].to(torch.int32).contiguous()
    rng = np.random.default_rng(cfg.seed)
    units = [(0, 0), (cfg.B - 1, cfg.H - 1)] + [(int(rng.integers(cfg.B)), int(rng.integers(cfg.H)))
                                                for _ in range(4)]
    assert check_case(marca, x, cfg.Nc, active, "bf16", units) == 0


@pytest.mark.parametrize("dtype,B,H,N", [("bf16", 2, 3, 320), ("bf16", 2, 3, 200),
                                         ("bf16", 3, 2, 77), ("bf16", 2, 2, 8),
                                         ("f32", 2, 2, 40), ("bf16", 128, 16, 320),
                                         # up to 64 tokens: the one-wave kernel, rows r -> r
                                         ("bf16", 2, 3, 40), ("bf16", 3, 2, 61)])
def test_fused_full_refresh(marca, dtype, B, H, N):
    """No active list: a refresh step's full attention over all N tokens and the
    rewrite of every cache row, in one call.  The output equals the plain full
    attention bit for bit, the caches equal the fresh K/V byte for byte, and
    sampled units match the oracle."""
    import oracle
    from mar_workloads import device_normal
    D = 64
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v, kc, vc = (device_normal((B, H, N, D), 300 + N + i, DEV, dt) for i in range(5))
    lse_ref = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    out_ref = marca.mar_cache_attn_fwd(q, k, v, kc, vc, None, Nc=0, lse=lse_ref)
    kc2, vc2 = kc.clone(), vc.clone()
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd_update(q, k, v, kc2, vc2, None, None, Nc=0, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
    assert np.array_equal(raw(kc2), raw(k)) and np.array_equal(raw(vc2), raw(v))
    for b, h in [(0, 0), (B - 1, H - 1)]:
        sl = lambda t: t[b:b + 1, h:h + 1].double().cpu().numpy()
        o, l = oracle.cache_attention(sl(q), sl(k), sl(v), sl(kc), sl(vc),
                                      np.zeros((1, 1), np.int32), D ** -0.5, Nc=0)
        got = out[b, h].double().cpu().numpy()
        if dtype == "bf16":
            assert np.abs(got - o[0, 0]).max() <= 2e-2
            assert np.abs(lse[b, h].double().cpu().numpy() - l[0, 0]).max() <= 4.5e-3
        else:
            assert np.abs(got - o[0, 0]).max() / np.abs(o[0, 0]).max() <= 1e-5
