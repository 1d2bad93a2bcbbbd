"""Edge cases at the documented limits of each entry point, against the oracle.

* attention: the largest token count the MFMA path takes (N = 8192, a 32 KB
  staged cached list), one past it (the row-wise path takes over), a cached
  list whose entries are all invalid, and a single (sequence, head) unit;
* full attention (no cached rows) over 4096 and 1088 tokens, several
  workgroups per unit with a partly idle last one, also with the full refresh;
* top-K: the largest N (4096, two-pass scores and LDS-read ranking), repeated
  G/P entries, every token taken (empty cached list);
* gate: a width above the multi-token kernel's range (one token per wave);
* scatter: every row rewritten through a permutation.
"""
import numpy as np
import pytest
import torch

from mar_workloads import Config, attention_inputs, device_normal, gate_features

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


def small_cfg(B, H, N, A, seed):
    return Config("t", B=B, H=H, D=64, N=N, n_prefix=0, A=A, n_gen=0, n_prev=0, K=0, layers=1,
                  dtype="bf16", stale=True, seed=seed)


def attn_vs_oracle(marca, x, Nc, cached, units, lse_tol=4.5e-3):
    import oracle
    B, H, A, D = x["q_a"].shape
    lse = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                   cached, Nc=Nc, lse=lse)
    torch.cuda.synchronize()
    cl = cached.cpu().numpy() if cached is not None else np.zeros((B, 1), np.int32)
    for b, h in units:
        sl = lambda t: f64(t[b:b + 1, h:h + 1])
        o, l = oracle.cache_attention(sl(x["q_a"]), sl(x["k_a"]), sl(x["v_a"]), sl(x["k_cache"]),
                                      sl(x["v_cache"]), cl[b:b + 1], D ** -0.5, Nc=Nc)
        assert np.abs(f64(out[b, h]) - o[0, 0]).max() <= 2e-2
        assert np.abs(f64(lse[b, h]) - l[0, 0]).max() <= lse_tol
    return out


@pytest.mark.parametrize("N,A", [(8192, 32), (8193, 32), (8192, 100)])
def test_attention_longest_sequences(marca, N, A):
    x = attention_inputs(small_cfg(1, 2, N, A, seed=N + A), DEV, ascending=False)
    attn_vs_oracle(marca, x, N - A, x["cached"], [(0, 0), (0, 1)])


def test_attention_all_cached_entries_invalid(marca):
    """Every list entry is out of range: the result is attention over the active rows."""
    x = attention_inputs(small_cfg(2, 2, 200, 48, seed=5), DEV)
    bad = torch.full((2, 152), -1, dtype=torch.int32, device=DEV)
    bad[:, ::3] = 200 + 7
    out = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"], bad,
                                   Nc=152)
    ref = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"], None,
                                   Nc=0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_attention_single_unit(marca):
    x = attention_inputs(small_cfg(1, 1, 320, 48, seed=9), DEV)
    attn_vs_oracle(marca, x, 272, x["cached"], [(0, 0)])


def test_topk_longest_sequence(marca):
    import oracle
    B, H, G, N = 1, 2, 16, 4096
    q = device_normal((B, H, G, 64), 41, DEV, torch.bfloat16)
    k = device_normal((B, H, N, 64), 42, DEV, torch.bfloat16)
    gp = torch.arange(0, 64, dtype=torch.int32, device=DEV)[None] * 7
    scores, act, cac, clen = marca.mar_refresh_topk(q, k, gp, 64, 100)
    torch.cuda.synchronize()
    s_ref = oracle.refresh_scores(f64(q), f64(k), 0.125)
    assert np.abs(f64(scores) - s_ref).max() / s_ref.max() <= 1e-5
    ra, rc, rl = oracle.refresh_select(f64(scores), gp.cpu().numpy(), 100, ld_cached=cac.shape[1])
    assert (act.cpu().numpy() == ra).all() and (cac.cpu().numpy() == rc).all()
    assert (clen.cpu().numpy() == rl).all() and int(clen[0]) == N - 64 - 100


def test_topk_repeated_entries_and_every_token_taken(marca):
    """Sequence 0: a G/P list of 20 entries with 5 repeats (15 distinct), K = 10,
    so 5 tokens stay cached; sequence 1: 20 distinct G/P tokens and K = 10 take
    all 30 tokens, leaving an empty cached list."""
    import oracle
    B, H, G, N, K = 2, 2, 4, 30, 10
    q = device_normal((B, H, G, 64), 43, DEV, torch.bfloat16)
    k = device_normal((B, H, N, 64), 44, DEV, torch.bfloat16)
    gp = torch.stack([torch.cat([torch.arange(15), torch.arange(5)]),
                      torch.arange(20)]).to(dtype=torch.int32, device=DEV)
    scores, act, cac, clen = marca.mar_refresh_topk(q, k, gp, 20, K)
    torch.cuda.synchronize()
    assert clen.cpu().numpy().tolist() == [5, 0]
    ra, rc, rl = oracle.refresh_select(f64(scores), gp.cpu().numpy(), K, ld_cached=cac.shape[1])
    assert (act.cpu().numpy() == ra).all() and (cac.cpu().numpy() == rc).all()
    assert (cac[1].cpu().numpy() == -1).all()


def test_gate_wide_features(marca):
    import oracle
    xc, yc, _ = gate_features(2, 40, 4096, seed=11, device=DEV)  # 512 pieces per token
    cos, reuse, cidx, clen = marca.mar_cos_gate(xc, yc, 0.95)
    torch.cuda.synchronize()
    c_ref, _, _, _ = oracle.cos_gate(f64(xc), f64(yc), 0.95)
    # the same bf16 values reduced in fp32 and fp64: chains of W/64 + 6 additions
    assert np.abs(f64(cos) - c_ref).max() <= 1e-5
    r2, c2, l2 = oracle.gate_from_cos(f64(cos), np.float32(0.95))
    assert (reuse.cpu().numpy() == r2).all() and (cidx.cpu().numpy() == c2).all()
    assert (clen.cpu().numpy() == l2).all()


def test_scatter_every_row(marca):
    import oracle
    B, H, N = 2, 3, 100
    kc = device_normal((B, H, N, 64), 51, DEV, torch.bfloat16)
    vc = device_normal((B, H, N, 64), 52, DEV, torch.bfloat16)
    kn = device_normal((B, H, N, 64), 53, DEV, torch.bfloat16)
    vn = device_normal((B, H, N, 64), 54, DEV, torch.bfloat16)
    g = torch.Generator().manual_seed(3)
    idx = torch.stack([torch.randperm(N, generator=g) for _ in range(B)]).to(torch.int32).to(DEV)
    raw = lambda t: t.cpu().view(torch.int16).numpy()
    rk, rv, skipped = oracle.kv_scatter(raw(kc), raw(vc), raw(kn), raw(vn), idx.cpu().numpy())
    k2, v2 = kc.clone(), vc.clone()
    marca.mar_kv_scatter_refresh(k2, v2, kn, vn, idx)
    torch.cuda.synchronize()
    assert skipped == 0
    assert np.array_equal(raw(k2), rk) and np.array_equal(raw(v2), rv)


@pytest.mark.parametrize("B,H,N,update", [(1, 2, 4096, False), (2, 2, 1088, False),
                                          (2, 2, 1088, True), (3, 1, 130, True)])
def test_full_attention_long_and_partial_blocks(marca, B, H, N, update):
    """All tokens active, no cached rows, more than one 320-query workgroup per
    (sequence, head) and a last workgroup with idle waves; with the full
    refresh the caches must become the fresh K/V exactly."""
    import oracle
    D = 64
    q, k, v, kc, vc = (device_normal((B, H, N, D), 700 + N + i, DEV, torch.bfloat16)
                       for i in range(5))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    if update:
        out = marca.mar_cache_attn_fwd_update(q, k, v, kc, vc, None, None, Nc=0, lse=lse)
    else:
        out = marca.mar_cache_attn_fwd(q, k, v, kc, vc, None, Nc=0, lse=lse)
    torch.cuda.synchronize()
    if update:
        assert torch.equal(kc, k) and torch.equal(vc, v)
    for b, h in [(0, 0), (B - 1, H - 1)]:
        sl = lambda t: f64(t[b:b + 1, h:h + 1])
        o, l = oracle.cache_attention(sl(q), sl(k), sl(v), sl(k), sl(v),
                                      np.zeros((1, 1), np.int32), D ** -0.5, Nc=0)
        assert np.abs(f64(out[b, h]) - o[0, 0]).max() <= 2e-2
        assert np.abs(f64(lse[b, h]) - l[0, 0]).max() <= 4.5e-3
