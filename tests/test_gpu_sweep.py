"""A seeded sweep of random shapes through every attention entry point, each
output checked against the oracle on every (sequence, head) unit.

The shapes are drawn once from a fixed seed (the list below is deterministic)
so that they land on every code path: the one-wave kernel with 1-4 query
tiles and one or several query groups, the dense workgroup kernel with full
and partial last chunks and partly idle workgroups, the row-wise path (A < 16),
empty and all-invalid cached lists, the fused cache update with a list and the
full refresh without one, and per-sequence counts.  Tolerances as everywhere:
bf16 max-abs 2e-2 (lse 4.5e-3), fp32 normwise 1e-5.
"""
import numpy as np
import pytest
import torch

from mar_workloads import device_normal

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _shapes(n, seed):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(g.integers(1, 4))
        H = int(g.integers(1, 4))
        N = int(g.integers(16, 700))
        kind = g.choice(["cached", "dense", "few_cached"])
        if kind == "dense":
            A, Nc = N, 0
        else:
            A = int(g.integers(16, N)) if N > 16 else 16
            Nc = N - A if kind == "cached" else int(g.integers(0, N - A + 1))
        out.append((B, H, N, A, Nc))
    return out


SHAPES = _shapes(24, 8080) + [(2, 2, 700, 8, 692), (1, 3, 64, 64, 0), (2, 1, 96, 96, 0),
                              (1, 2, 65, 65, 0), (3, 1, 200, 33, 0)]


@pytest.fixture(scope="module")
def marca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_attention_amd as m
    return m


def f64(t):
    return t.detach().double().cpu().numpy()


def raw(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy()


def inputs(B, H, N, A, Nc, seed, dt=torch.bfloat16):
    q, ka, va = (device_normal((B, H, A, 64), seed + i, DEV, dt) for i in range(3))
    kc, vc = (device_normal((B, H, N, 64), seed + 3 + i, DEV, dt) for i in range(2))
    g = torch.Generator().manual_seed(seed)
    perms = [torch.randperm(N, generator=g) for _ in range(B)]
    active = torch.stack([p[:A] for p in perms]).to(torch.int32).to(DEV)
    cached = torch.stack([p[A:A + max(Nc, 1)] if A + max(Nc, 1) <= N else
                          torch.cat([p[A:], torch.full((A + 1 - N,), -1)]) for p in perms])
    cached = cached.to(torch.int32).to(DEV)
    return q, ka, va, kc, vc, active, cached


def oracle_units(q, ka, va, kc, vc, cached, Nc, out, lse, an=None, cn=None, tol=2e-2):
    import oracle
    B, H, A, D = q.shape
    cl_all = cached.cpu().numpy()
    for b in range(B):
        a_b = A if an is None else int(an[b])
        c_b = Nc if cn is None else int(cn[b])
        if a_b == 0:
            continue
        for h in range(H):
            sl = lambda t, n: f64(t[b:b + 1, h:h + 1, :n])
            o, l = oracle.cache_attention(sl(q, a_b), sl(ka, a_b), sl(va, a_b),
                                          f64(kc[b:b + 1, h:h + 1]), f64(vc[b:b + 1, h:h + 1]),
                                          cl_all[b:b + 1, :max(c_b, 1)], D ** -0.5, Nc=c_b)
            got = f64(out[b, h, :a_b])
            if q.dtype == torch.bfloat16:
                assert np.abs(got - o[0, 0]).max() <= tol, (b, h)
                if lse is not None:
                    assert np.abs(f64(lse[b, h, :a_b]) - l[0, 0]).max() <= 4.5e-3, (b, h)
            else:
                assert np.abs(got - o[0, 0]).max() / np.abs(o[0, 0]).max() <= 1e-5, (b, h)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dN%dA%dNc%d" % s)
def test_sweep_attention_and_fused_update(marca, shape):
    B, H, N, A, Nc = shape
    seed = 100 * N + A
    q, ka, va, kc, vc, active, cached = inputs(B, H, N, A, Nc, seed)
    cl = cached if Nc > 0 else None
    lse = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(q, ka, va, kc, vc, cl, Nc=Nc, lse=lse)
    torch.cuda.synchronize()
    oracle_units(q, ka, va, kc, vc, cached, Nc, out, lse)

    # the fused cache update: same output bits, active rows written
    import oracle
    kc2, vc2 = kc.clone(), vc.clone()
    out2 = marca.mar_cache_attn_fwd_update(q, ka, va, kc2, vc2, cl, active, Nc=Nc)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    kr, vr, skipped = oracle.kv_scatter(raw(kc), raw(vc), raw(ka), raw(va), active.cpu().numpy())
    assert skipped == 0
    assert np.array_equal(raw(kc2), kr) and np.array_equal(raw(vc2), vr)

    if A == N and Nc == 0:  # the full refresh: no list, every row rewritten
        kc3, vc3 = kc.clone(), vc.clone()
        out3 = marca.mar_cache_attn_fwd_update(q, ka, va, kc3, vc3, None, None, Nc=0)
        torch.cuda.synchronize()
        assert torch.equal(out3, out)
        assert torch.equal(kc3, ka) and torch.equal(vc3, va)


@pytest.mark.parametrize("shape", [s for s in SHAPES if s[4] > 0][:10],
                         ids=lambda s: "B%dH%dN%dA%dNc%d" % s)
def test_sweep_ragged(marca, shape):
    B, H, N, A, Nc = shape
    seed = 7 * N + A
    q, ka, va, kc, vc, active, cached = inputs(B, H, N, A, Nc, seed)
    g = np.random.default_rng(seed)
    an = g.integers(0, A + 1, size=B).astype(np.int32)
    cn = g.integers(0, Nc + 1, size=B).astype(np.int32)
    a_len = torch.from_numpy(an).to(DEV)
    c_len = torch.from_numpy(cn).to(DEV)
    out = torch.full((B, H, A, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    marca.mar_cache_attn_fwd_ragged(q, ka, va, kc, vc, cached, a_len, c_len, out=out)
    torch.cuda.synchronize()
    for b in range(B):
        assert (out[b, :, int(an[b]):].float() == 3.0).all()
    oracle_units(q, ka, va, kc, vc, cached, Nc, out, None, an=an, cn=cn)


@pytest.mark.parametrize("shape", [(2, 2, 100, 40, 60), (1, 2, 300, 300, 0), (2, 1, 50, 7, 43)])
def test_sweep_fp32(marca, shape):
    B, H, N, A, Nc = shape
    q, ka, va, kc, vc, active, cached = inputs(B, H, N, A, Nc, 11 * N, torch.float32)
    out = marca.mar_cache_attn_fwd(q, ka, va, kc, vc, cached if Nc > 0 else None, Nc=Nc)
    torch.cuda.synchronize()
    oracle_units(q, ka, va, kc, vc, cached, Nc, out, None)
