"""GPU parity of mar_cache_attn_fwd_ragged (per-sequence active / cached set
sizes) against the oracle, and the LazyMAR token-cache chain: the cosine gate
picks each sequence's tokens to recompute, and the attention runs over those
fresh rows plus the reused cached rows of the other tokens.

Tolerances as for mar_cache_attn_fwd (bf16: max-abs 2e-2; fp32: normwise 1e-5).
Rows past a sequence's active count must be left untouched.
"""
import numpy as np
import pytest
import torch

from mar_workloads import device_normal, gate_features

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


def oracle_seq(q, ka, va, kc, vc, cached, b, h, an, cn, scale):
    import oracle
    sl = lambda t, n: f64(t[b:b + 1, h:h + 1, :n])
    cl = cached[b:b + 1, :max(cn, 1)].cpu().numpy()
    o, l = oracle.cache_attention(sl(q, an), sl(ka, an), sl(va, an), f64(kc[b:b + 1, h:h + 1]),
                                  f64(vc[b:b + 1, h:h + 1]), cl, scale, Nc=cn)
    return o[0, 0], l[0, 0]


@pytest.mark.parametrize("dtype,A,Nc", [("bf16", 64, 250), ("bf16", 100, 200), ("f32", 40, 120),
                                        ("bf16", 12, 90), ("bf16", 200, 700), ("bf16", 256, 500)])
def test_ragged_lengths(marca, dtype, A, Nc):
    B, H, N, D = 5, 2, A + Nc + 10, 64
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = device_normal((B, H, A, D), 1, DEV, dt)
    ka = device_normal((B, H, A, D), 2, DEV, dt)
    va = device_normal((B, H, A, D), 3, DEV, dt)
    kc = device_normal((B, H, N, D), 4, DEV, dt)
    vc = device_normal((B, H, N, D), 5, DEV, dt)
    g = torch.Generator().manual_seed(A + Nc)
    cached = torch.stack([torch.randperm(N, generator=g)[:Nc] for _ in range(B)]).to(
        dtype=torch.int32, device=DEV)
    a_len = torch.tensor([A, 0, A // 2 + 1, 1, A - 3], dtype=torch.int32, device=DEV)
    c_len = torch.tensor([Nc, Nc // 3, 0, Nc, 5], dtype=torch.int32, device=DEV)
    lse = torch.full((B, H, A), 7.0, dtype=torch.float32, device=DEV)
    out = torch.full((B, H, A, D), 3.0, dtype=dt, device=DEV)
    marca.mar_cache_attn_fwd_ragged(q, ka, va, kc, vc, cached, a_len, c_len, out=out, lse=lse)
    torch.cuda.synchronize()
    for b in range(B):
        an, cn = int(a_len[b]), int(c_len[b])
        # rows past the active count are untouched
        assert (out[b, :, an:].float() == 3.0).all() and (lse[b, :, an:] == 7.0).all()
        if an == 0:
            continue
        for h in range(H):
            o, l = oracle_seq(q, ka, va, kc, vc, cached, b, h, an, cn, D ** -0.5)
            got = f64(out[b, h, :an])
            if dtype == "bf16":
                assert np.abs(got - o).max() <= 2e-2, (b, h)
                assert np.abs(f64(lse[b, h, :an]) - l).max() <= 4.5e-3
            else:
                assert np.abs(got - o).max() / np.abs(o).max() <= 1e-5, (b, h)


def test_full_lengths_match_mar_cache_attn_fwd(marca):
    B, H, A, Nc, N = 3, 4, 48, 272, 320
    t = [device_normal(s, 10 + i, DEV, torch.bfloat16) for i, s in enumerate(
        [(B, H, A, 64)] * 3 + [(B, H, N, 64)] * 2)]
    g = torch.Generator().manual_seed(0)
    cached = torch.stack([torch.randperm(N, generator=g)[:Nc] for _ in range(B)]).to(
        dtype=torch.int32, device=DEV)
    full = marca.mar_cache_attn_fwd(*t, cached)
    a_len = torch.full((B,), A, dtype=torch.int32, device=DEV)
    c_len = torch.full((B,), Nc, dtype=torch.int32, device=DEV)
    rag = marca.mar_cache_attn_fwd_ragged(*t, cached, a_len, c_len)
    torch.cuda.synchronize()
    assert torch.equal(full, rag)


def test_lazymar_token_cache_chain(marca):
    """Gate -> per-sequence recompute sets -> ragged cache-aware attention."""
    B, H, N, D, W = 4, 2, 320, 64, 256
    xg, yg, _ = gate_features(B, N, W, seed=21, device=DEV)
    cos, reuse, cidx, clen = marca.mar_cos_gate(xg, yg, 0.95)
    # fresh Q/K/V of every token now, stale K/V of every token in the cache
    qf = device_normal((B, H, N, D), 31, DEV, torch.bfloat16)
    kf = device_normal((B, H, N, D), 32, DEV, torch.bfloat16)
    vf = device_normal((B, H, N, D), 33, DEV, torch.bfloat16)
    kc = device_normal((B, H, N, D), 34, DEV, torch.bfloat16)
    vc = device_normal((B, H, N, D), 35, DEV, torch.bfloat16)
    torch.cuda.synchronize()
    n_comp = clen.cpu().numpy()
    A = int(n_comp.max())
    assert 0 < A < N
    comp = cidx[:, :A].clamp(min=0).long()  # recompute positions (padding rows unused)
    gat = lambda x: torch.gather(x, 2, comp[:, None, :, None].expand(B, H, A, D)).contiguous()
    q_a, k_a, v_a = gat(qf), gat(kf), gat(vf)
    reuse_pos = [torch.nonzero(reuse[b]).flatten().to(torch.int32) for b in range(B)]
    Nc = max(len(r) for r in reuse_pos)
    cached = torch.full((B, Nc), -1, dtype=torch.int32, device=DEV)
    for b in range(B):
        cached[b, :len(reuse_pos[b])] = reuse_pos[b]
    c_len = torch.tensor([len(r) for r in reuse_pos], dtype=torch.int32, device=DEV)
    assert ((c_len + clen) == N).all()
    out = marca.mar_cache_attn_fwd_ragged(q_a, k_a, v_a, kc, vc, cached, clen, c_len)
    torch.cuda.synchronize()
    for b in range(B):
        an, cn = int(n_comp[b]), int(c_len[b])
        for h in range(H):
            o, _ = oracle_seq(q_a, k_a, v_a, kc, vc, cached, b, h, an, cn, D ** -0.5)
            assert np.abs(f64(out[b, h, :an]) - o).max() <= 2e-2, (b, h)


def raw(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy()


@pytest.mark.parametrize("B,H,A,Nc", [(5, 2, 64, 250), (5, 2, 100, 200), (5, 2, 200, 700),
                                      (1, 2, 40, 300)])
def test_ragged_update(marca, B, H, A, Nc):
    """mar_cache_attn_fwd_ragged_update: the output of mar_cache_attn_fwd_ragged
    bit for bit, and each sequence's first a_len[b] fresh rows written into the
    caches at active_idx (the oracle's scatter on the list cut at a_len[b]);
    entries past a_len[b] are padding that is never read, and a bad entry
    before it is skipped and counted once per sequence.  The shapes take the
    one-wave kernel (64 queries), the cached workgroup kernel with two and with
    four waves, and the split kernel (two units)."""
    import oracle
    D = 64
    N = A + Nc + 10
    q, ka, va = (device_normal((B, H, A, D), 40 + i, DEV, torch.bfloat16) for i in range(3))
    kc, vc = (device_normal((B, H, N, D), 50 + i, DEV, torch.bfloat16) for i in range(2))
    g = torch.Generator().manual_seed(A * 7 + Nc)
    a_len = torch.tensor([A, 0, A // 2 + 1, 1, A - 3][:B], dtype=torch.int32)
    c_len = torch.tensor([Nc, Nc // 3, 0, Nc, 5][:B], dtype=torch.int32)
    act = torch.full((B, A + 3), -1, dtype=torch.int32)      # ld_act > A
    cached = torch.full((B, Nc), -1, dtype=torch.int32)
    bad = 0
    for b in range(B):
        perm = torch.randperm(N, generator=g).to(torch.int32)
        an = int(a_len[b])
        act[b, :A] = perm[:A]
        cached[b] = perm[A:A + Nc]
        act[b, an:A] = 77777  # padding past the sequence's count: never read
        if b == 0 and an > 3:
            act[b, 2] = N + 5  # a bad entry before the count: skipped, counted
            bad += 1
    act_d, cached_d = act.to(DEV), cached.to(DEV)
    a_d, c_d = a_len.to(DEV), c_len.to(DEV)
    ref = marca.mar_cache_attn_fwd_ragged(q, ka, va, kc, vc, cached_d, a_d, c_d)
    k0, v0 = raw(kc), raw(vc)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = marca.mar_cache_attn_fwd_ragged_update(q, ka, va, kc, vc, cached_d, act_d, a_d, c_d,
                                                 err_count=err)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    idx = act[:, :A].clone()
    for b in range(B):
        idx[b, int(a_len[b]):] = -1
    kr, vr, skipped = oracle.kv_scatter(k0, v0, raw(ka), raw(va), idx.numpy())
    assert np.array_equal(raw(kc), kr) and np.array_equal(raw(vc), vr)
    assert int(err.item()) == bad
    assert skipped == bad + int((A - a_len).sum())
    # the attention itself against the oracle on one sampled head per sequence
    for b in range(B):
        an, cn = int(a_len[b]), int(c_len[b])
        if an == 0:
            continue
        o, _ = oracle_seq(q, ka, va, torch.from_numpy(k0).view(torch.bfloat16).to(DEV),
                          torch.from_numpy(v0).view(torch.bfloat16).to(DEV), cached_d, b, b % H,
                          an, cn, D ** -0.5)
        assert np.abs(f64(out[b, b % H, :an]) - o).max() <= 2e-2, b


def test_ragged_update_full_size_gated_layer(marca):
    """A high-res gated layer at full size, as the high-res decode runs it: 64
    sequences x 16 heads x 1088 tokens, the token gate (W = 1024, 0.95) picks
    each sequence's tokens to recompute, and mar_cache_attn_fwd_ragged_update
    attends their fresh rows over the cached rows of the reused tokens and
    writes the fresh rows into the caches.  Checked: the output equals
    mar_cache_attn_fwd_ragged's bit for bit, every recomputed row of every
    head is written and no other row changes (sampled sequences), and sampled
    (sequence, head) units match the oracle."""
    from mar_workloads import device_gate_features
    B, H, N, D, W = 64, 16, 1088, 64, 1024
    gx, gy, _ = device_gate_features(B, N, W, seed=77, device=DEV)
    reuse_idx = torch.empty((B, N), dtype=torch.int32, device=DEV)
    reuse_len = torch.empty((B,), dtype=torch.int32, device=DEV)
    _, _, comp, clen = marca.mar_cos_gate(gx, gy, 0.95, reuse_idx=reuse_idx, reuse_len=reuse_len)
    del gx, gy
    torch.cuda.synchronize()
    a_cap = int(clen.max())
    nc_cap = int(reuse_len.max())
    assert 100 < a_cap < N and ((clen + reuse_len) == N).all()
    qf, kf, vf = (device_normal((B, H, N, D), 60 + i, DEV, torch.bfloat16) for i in range(3))
    kc, vc = (device_normal((B, H, N, D), 70 + i, DEV, torch.bfloat16) for i in range(2))
    pos = comp[:, :a_cap].clamp(min=0).long()
    gat = lambda x: torch.gather(x, 2, pos[:, None, :, None].expand(B, H, a_cap, D)).contiguous()
    q_a, k_a, v_a = gat(qf), gat(kf), gat(vf)
    del qf, kf, vf
    active = comp[:, :a_cap].contiguous()
    cached = reuse_idx[:, :nc_cap].contiguous()
    ref = marca.mar_cache_attn_fwd_ragged(q_a, k_a, v_a, kc, vc, cached, clen, reuse_len)
    torch.cuda.synchronize()
    samples = (0, 17, 40, B - 1)
    before_k = {b: kc[b].clone() for b in samples}
    before_v = {b: vc[b].clone() for b in samples}
    out = marca.mar_cache_attn_fwd_ragged_update(q_a, k_a, v_a, kc, vc, cached, active, clen,
                                                 reuse_len)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    for b in samples:
        an = int(clen[b])
        rows = comp[b, :an].long()
        assert torch.equal(kc[b][:, rows], k_a[b, :, :an]) and torch.equal(vc[b][:, rows], v_a[b, :, :an])
        keep = torch.ones(N, dtype=torch.bool, device=DEV)
        keep[rows] = False
        assert torch.equal(kc[b][:, keep], before_k[b][:, keep])
        assert torch.equal(vc[b][:, keep], before_v[b][:, keep])
    for b, h in ((0, 0), (17, 5), (40, 15), (B - 1, 9)):
        an, cn = int(clen[b]), int(reuse_len[b])
        o, _ = oracle_seq(q_a, k_a, v_a, before_k[b][None].expand(B, H, N, D),
                          before_v[b][None].expand(B, H, N, D), cached, b, h, an, cn, D ** -0.5)
        assert np.abs(f64(out[b, h, :an]) - o).max() <= 2e-2, (b, h)
