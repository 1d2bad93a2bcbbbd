"""GPU parity of the fp32 matrix-core attention (fp32 inputs, 16 or more
active queries) against the CPU oracle.

Tolerance: normwise relative error max|g - r| / max|r| <= 1e-5 per (sequence,
head) tile on the outputs, 1e-5 relative on the log-sum-exp (the accuracy
target for fp32).  The products run on v_mfma_f32_16x16x4_f32 with fp32
accumulation and the probabilities stay in fp32, so the error is a few fp32
roundings per score and per output element.

Covered: the query tile counts 1-4 and two query groups, partial last tiles
and chunks, an empty and a one-entry cached list, invalid list entries, the
softmax rescale path (scores that climb along the sequence), per-sequence
counts (including sequences with no queries, left untouched), the fused cache
update (attention + row scatter, same output bits), the longest sequence the
path takes (8192 tokens) and one past it, an all-invalid list, and the MAR-L
shape at full size on sampled units.
"""
import numpy as np
import pytest
import torch

from mar_workloads import CONFIGS, Config, attention_inputs, device_normal

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


def oracle_unit(q, ka, va, kc, vc, cached, b, h, an, cn):
    import oracle
    sl = lambda t, n=None: f64(t[b:b + 1, h:h + 1] if n is None else t[b:b + 1, h:h + 1, :n])
    cl = cached[b:b + 1, :max(cn, 1)].cpu().numpy() if cached is not None else np.zeros((1, 1), np.int32)
    o, l = oracle.cache_attention(sl(q, an), sl(ka, an), sl(va, an), sl(kc), sl(vc), cl,
                                  q.shape[-1] ** -0.5, Nc=cn)
    return o[0, 0], l[0, 0]


def check_unit(out, lse, ref_o, ref_l, what):
    got = f64(out)
    err = np.abs(got - ref_o).max() / np.abs(ref_o).max()
    assert err <= 1e-5, f"{what}: normwise error {err}"
    np.testing.assert_allclose(f64(lse), ref_l, rtol=1e-5, atol=1e-6, err_msg=str(what))


def small_cfg(B, H, N, A, seed):
    return Config("t", B=B, H=H, D=64, N=N, n_prefix=0, A=A, n_gen=0, n_prev=0, K=0, layers=1,
                  dtype="f32", stale=True, seed=seed)


@pytest.mark.parametrize("A,Nc", [(16, 0), (16, 48), (17, 31), (24, 296), (33, 1), (48, 272),
                                  (64, 256), (65, 100), (100, 37), (128, 160)])
def test_f32_mfma_shapes(marca, A, Nc):
    cfg = small_cfg(B=2, H=3, N=A + Nc + 5, A=A, seed=7000 + A * 10 + Nc)
    x = attention_inputs(cfg, DEV, ascending=False)
    B, H = 2, 3
    lse = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                   x["cached"], Nc=Nc, lse=lse)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            o, l = oracle_unit(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                               x["cached"], b, h, A, Nc)
            check_unit(out[b, h], lse[b, h], o, l, (A, Nc, b, h))


def test_f32_invalid_list_entries(marca):
    """-1 padding and out-of-range entries are skipped, as if absent."""
    A, N, B, H = 40, 200, 2, 2
    cfg = small_cfg(B=B, H=H, N=N, A=A, seed=7101)
    x = attention_inputs(cfg, DEV)
    cached = x["cached"].cpu().numpy()
    Nc = cached.shape[1]
    bad = np.full((B, N), -1, np.int32)
    bad[:, :Nc] = cached
    bad[:, 3] = N + 11
    bad[:, 40] = -5
    out = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                   torch.from_numpy(bad).to(DEV), Nc=Nc)
    torch.cuda.synchronize()
    keep = torch.from_numpy(np.delete(cached, [3, 40], axis=1))
    for b, h in ((0, 0), (1, 1)):
        o, _ = oracle_unit(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"], keep, b, h,
                           A, Nc - 2)
        err = np.abs(f64(out[b, h]) - o).max() / np.abs(o).max()
        assert err <= 1e-5, (b, h, err)


@pytest.mark.parametrize("A", [48, 128])
def test_f32_rising_scores(marca, A):
    """Key rows grow along the sequence, so every query's maximum climbs far
    past its first chunk's and the state is rescaled many times."""
    B, H, N = 6, 4, 320
    Nc = N - A
    q, ka, va = (device_normal((B, H, A, 64), 7200 + i, DEV, torch.float32) for i in range(3))
    kc, vc = (device_normal((B, H, N, 64), 7210 + i, DEV, torch.float32) for i in range(2))
    ramp = (1.0 + 3.0 * torch.arange(N, dtype=torch.float32, device=DEV) / N)[None, None, :, None]
    q, ka, kc = q * 2.0, ka * 2.0, kc * ramp * 2.0
    s = (q[0, 0] @ kc[0, 0].t()) / 8.0
    assert (s[:, -32:].max(1).values - s[:, :32].max(1).values).max() * 1.4427 > 16
    g = torch.Generator().manual_seed(A)
    cached = torch.stack([torch.sort(torch.randperm(N, generator=g)[:Nc]).values
                          for _ in range(B)]).to(torch.int32).to(DEV)
    lse = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(q, ka, va, kc, vc, cached, Nc=Nc, lse=lse)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1), (2, 1)):
        o, l = oracle_unit(q, ka, va, kc, vc, cached, b, h, A, Nc)
        check_unit(out[b, h], lse[b, h], o, l, (A, b, h))


@pytest.mark.parametrize("A,Nc", [(48, 272), (100, 200)])
def test_f32_ragged_counts(marca, A, Nc):
    B, H, N, D = 5, 2, A + Nc + 10, 64
    q, ka, va = (device_normal((B, H, A, D), 7300 + i, DEV, torch.float32) for i in range(3))
    kc, vc = (device_normal((B, H, N, D), 7310 + i, DEV, torch.float32) for i in range(2))
    g = torch.Generator().manual_seed(A + Nc)
    cached = torch.stack([torch.randperm(N, generator=g)[:Nc] for _ in range(B)]).to(
        dtype=torch.int32, device=DEV)
    a_len = torch.tensor([A, 0, A // 2 + 1, 16, A - 3], dtype=torch.int32, device=DEV)
    c_len = torch.tensor([Nc, Nc // 3, 0, Nc, 5], dtype=torch.int32, device=DEV)
    lse = torch.full((B, H, A), 7.0, dtype=torch.float32, device=DEV)
    out = torch.full((B, H, A, D), 3.0, dtype=torch.float32, device=DEV)
    marca.mar_cache_attn_fwd_ragged(q, ka, va, kc, vc, cached, a_len, c_len, out=out, lse=lse)
    torch.cuda.synchronize()
    for b in range(B):
        an, cn = int(a_len[b]), int(c_len[b])
        assert (out[b, :, an:] == 3.0).all() and (lse[b, :, an:] == 7.0).all(), b
        for h in range(H if an else 0):
            o, l = oracle_unit(q, ka, va, kc, vc, cached, b, h, an, cn)
            check_unit(out[b, h, :an], lse[b, h, :an], o, l, (b, h))


def test_f32_update_same_bits_and_rows_written(marca):
    B, H, A, N = 3, 4, 48, 320
    Nc = N - A
    q, ka, va = (device_normal((B, H, A, 64), 7400 + i, DEV, torch.float32) for i in range(3))
    kc, vc = (device_normal((B, H, N, 64), 7410 + i, DEV, torch.float32) for i in range(2))
    g = torch.Generator().manual_seed(5)
    perm = torch.stack([torch.randperm(N, generator=g) for _ in range(B)]).to(torch.int32)
    active, cached = perm[:, :A].contiguous().to(DEV), perm[:, A:].contiguous().to(DEV)
    lse = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(q, ka, va, kc, vc, cached, Nc=Nc, lse=lse)
    kc2, vc2 = kc.clone(), vc.clone()
    lse2 = torch.empty_like(lse)
    out2 = marca.mar_cache_attn_fwd_update(q, ka, va, kc2, vc2, cached, active, Nc=Nc, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)
    ak = active.long()[:, None, :, None].expand(B, H, A, 64)
    assert torch.equal(torch.gather(kc2, 2, ak), ka) and torch.equal(torch.gather(vc2, 2, ak), va)
    # the cached rows are untouched
    ck = cached.long()[:, None, :, None].expand(B, H, Nc, 64)
    assert torch.equal(torch.gather(kc2, 2, ck), torch.gather(kc, 2, ck))


def test_f32_full_size_mar_l_sampled(marca):
    """The MAR-L shape (128 sequences x 16 heads, 48 active, 272 cached) in
    fp32, as the bench times it: sampled units against the oracle."""
    base = CONFIGS["mar_l"]
    cfg = base.__class__(**{**base.__dict__, "dtype": "f32"})
    x = attention_inputs(cfg, DEV, seed=cfg.seed * 100 + 50)
    B, H, A = cfg.B, cfg.H, cfg.A
    lse = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                   x["cached"], Nc=cfg.Nc, lse=lse)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1), (37, 5), (64, 15), (101, 8), (127, 0)):
        o, l = oracle_unit(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"], x["cached"],
                           b, h, A, cfg.Nc)
        check_unit(out[b, h], lse[b, h], o, l, (b, h))


@pytest.mark.parametrize("N,A", [(8192, 32), (8193, 32)])
def test_f32_longest_sequences(marca, N, A):
    """The largest token count the fp32 matrix-core path takes (a 32 KB staged
    list) and one past it, where the per-unit vector path takes over."""
    cfg = small_cfg(B=1, H=2, N=N, A=A, seed=7500 + N)
    x = attention_inputs(cfg, DEV, ascending=False)
    lse = torch.empty((1, 2, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                   x["cached"], Nc=N - A, lse=lse)
    torch.cuda.synchronize()
    for h in range(2):
        o, l = oracle_unit(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"], x["cached"],
                           0, h, A, N - A)
        check_unit(out[0, h], lse[0, h], o, l, (N, h))


def test_f32_all_cached_entries_invalid(marca):
    """Every list entry is out of range: the same bits as attention over the
    active rows alone."""
    cfg = small_cfg(B=2, H=2, N=200, A=48, seed=7600)
    x = attention_inputs(cfg, DEV)
    bad = torch.full((2, 152), -1, dtype=torch.int32, device=DEV)
    bad[:, ::3] = 200 + 7
    out = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"], bad,
                                   Nc=152)
    ref = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"], None,
                                   Nc=0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
