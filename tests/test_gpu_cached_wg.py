"""GPU parity of the workgroup path of cache-aware attention: with more than 64
active queries per (sequence, head) unit and many units, the library runs one
workgroup per unit (per block of 128 or 256 of its queries) whose waves share
each K/V chunk of the unit's [active ; cached] sequence through LDS.

Each case draws two sequences x two heads and tiles them into a batch of 160
sequences (320 units, enough for this path), runs the batch once, checks that
every copy computed the same thing, and checks the first two sequences
against the oracle (bf16 max-abs 2e-2, log-sum-exp 4.5e-3).  The cases cover a
complete and a ragged last chunk, query counts that leave partial query tiles
and idle waves, two and four waves per workgroup, two query blocks per unit,
and skipped cached entries (-1 and past N), which send their chunks down the
masked path.  The fused cache update must give the same output bits, write
the active rows exactly once (only the unit's first block writes) and count
each skipped active entry once per sequence.
"""
import numpy as np
import pytest
import torch

from mar_workloads import device_normal

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
TILE = 80

# (N, A, Nc, skipped cached entries per sequence)
CASES = [(1088, 128, 960, 0),   # the high-res layer: 2 waves, 34 complete chunks
         (400, 100, 270, 0),    # T = 370: a ragged last chunk; 36 queries in the second wave
         (700, 65, 600, 9),     # skipped entries: masked chunks; a 1-query tile
         (900, 200, 650, 0),    # 4 waves, the last with 8 queries
         (1200, 300, 880, 5),   # 2 blocks of 256 queries per unit
         # The active rows fill ceil(A/32) chunks and the cached rows start on the
         # next one, so the staged lists need ceil(A/32) + ceil(Nc/32) chunk masks.
         # Here the staged lists take exactly 128 entries (512 bytes, no rounding
         # slack) and that count is one more than ceil((A + Nc)/32).
         (300, 100, 121, 0)]


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


def case(N, A, Nc, n_skip, seed):
    B, H = 2, 2
    q, ka, va = (device_normal((B, H, A, 64), seed + i, DEV, torch.bfloat16) for i in range(3))
    kc, vc = (device_normal((B, H, N, 64), seed + 3 + i, DEV, torch.bfloat16) for i in range(2))
    g = torch.Generator().manual_seed(seed)
    perms = [torch.randperm(N, generator=g) for _ in range(B)]
    active = torch.stack([p[:A] for p in perms]).to(torch.int32)
    cached = torch.stack([p[A:A + Nc] for p in perms]).to(torch.int32)
    if n_skip:
        pos = torch.randperm(Nc, generator=g)[:n_skip]
        cached[0, pos[::2]] = -1
        cached[0, pos[1::2]] = N + 5
    tile = lambda t: t.repeat(TILE, *([1] * (t.dim() - 1))).contiguous()
    return [tile(t) for t in (q, ka, va, kc, vc)], tile(active).to(DEV), tile(cached).to(DEV)


def check_oracle(ts, cached, Nc, out, lse):
    """The library skips a cached entry outside [0, N); the oracle takes the
    list without it."""
    import oracle
    q, ka, va, kc, vc = ts
    N = kc.shape[2]
    cl = cached.cpu().numpy()
    for b in range(2):
        keep = cl[b, :Nc][(cl[b, :Nc] >= 0) & (cl[b, :Nc] < N)][None, :]
        for h in range(2):
            sl = lambda t: f64(t[b:b + 1, h:h + 1])
            o, l = oracle.cache_attention(sl(q), sl(ka), sl(va), sl(kc), sl(vc), keep, 0.125,
                                          Nc=keep.shape[1])
            assert np.abs(f64(out[b, h]) - o[0, 0]).max() <= 2e-2, (b, h)
            assert np.abs(f64(lse[b, h]) - l[0, 0]).max() <= 4.5e-3, (b, h)


@pytest.mark.parametrize("N,A,Nc,n_skip", CASES)
def test_cached_workgroup_attention(marca, N, A, Nc, n_skip):
    ts, active, cached = case(N, A, Nc, n_skip, seed=7 * N + A)
    B = ts[0].shape[0]
    lse = torch.empty((B, 2, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(*ts, cached, Nc=Nc, lse=lse)
    torch.cuda.synchronize()
    for t in range(1, TILE):
        assert torch.equal(out[2 * t:2 * t + 2], out[:2])
    check_oracle(ts, cached, Nc, out, lse)


@pytest.mark.parametrize("N,A,Nc,n_skip", [CASES[0], CASES[2], CASES[4],
                                            (200, 100, 24, 0)])  # lists + masks: 128 entries
def test_cached_workgroup_fused_update(marca, N, A, Nc, n_skip):
    import oracle
    ts, active, cached = case(N, A, Nc, n_skip, seed=11 * N + A)
    q, ka, va, kc, vc = ts
    B = q.shape[0]
    # two skipped active entries in the first sequence (each copy of it)
    active[0::2, 3] = -1
    active[0::2, A - 1] = N
    out = marca.mar_cache_attn_fwd(*ts, cached, Nc=Nc)
    kc2, vc2 = kc.clone(), vc.clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out2 = marca.mar_cache_attn_fwd_update(q, ka, va, kc2, vc2, cached, active, Nc=Nc,
                                           err_count=err)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    # once per sequence (not per head): 2 per copy of the first sequence
    assert int(err.item()) == 2 * TILE
    kr, vr, skipped = oracle.kv_scatter(raw(kc[:2]), raw(vc[:2]), raw(ka[:2]), raw(va[:2]),
                                        active[:2].cpu().numpy())
    assert skipped == 2
    assert np.array_equal(raw(kc2[:2]), kr) and np.array_equal(raw(vc2[:2]), vr)
    for t in range(1, TILE):
        assert torch.equal(kc2[2 * t:2 * t + 2], kc2[:2]) and torch.equal(vc2[2 * t:2 * t + 2], vc2[:2])


@pytest.mark.parametrize("N,A,Nc,n_skip", [CASES[0], (700, 200, 480, 9), CASES[4]])
def test_cached_workgroup_ragged(marca, N, A, Nc, n_skip):
    """Per-sequence counts (LazyMAR's token cache): A and Nc are capacities;
    rows past a sequence's active count stay untouched, a sequence with no
    active rows writes nothing, and a block whose queries all lie past the
    count returns at once."""
    import oracle
    ts, active, cached = case(N, A, Nc, n_skip, seed=13 * N + A)
    B = ts[0].shape[0]
    for an, cn in [(A, Nc), (0, Nc), (1, 0), (20, 7), (A // 2 + 3, Nc - 33), (A - 1, Nc)]:
        a_len = torch.tensor([an, A - 5], dtype=torch.int32, device=DEV).repeat(TILE)
        c_len = torch.tensor([cn, Nc // 2], dtype=torch.int32, device=DEV).repeat(TILE)
        out = torch.full((B, 2, A, 64), 3.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, 2, A), 7.0, dtype=torch.float32, device=DEV)
        marca.mar_cache_attn_fwd_ragged(*ts, cached, a_len, c_len, out=out, lse=lse)
        torch.cuda.synchronize()
        for t in range(1, TILE):
            assert torch.equal(out[2 * t:2 * t + 2], out[:2]), (an, cn)
        assert (out[0, :, an:].float() == 3.0).all() and (lse[0, :, an:] == 7.0).all()
        assert (out[1, :, A - 5:].float() == 3.0).all()
        q, ka, va, kc, vc = ts
        cl = cached.cpu().numpy()
        for b, (a_b, c_b) in enumerate([(an, cn), (A - 5, Nc // 2)]):
            if a_b == 0:
                continue
            keep = cl[b, :c_b][(cl[b, :c_b] >= 0) & (cl[b, :c_b] < N)][None, :]
            for h in range(2):
                sl = lambda t, n=None: f64(t[b:b + 1, h:h + 1, :n])
                o, l = oracle.cache_attention(sl(q, a_b), sl(ka, a_b), sl(va, a_b), sl(kc), sl(vc),
                                              keep if keep.size else np.zeros((1, 1), np.int32),
                                              0.125, Nc=keep.shape[1])
                assert np.abs(f64(out[b, h, :a_b]) - o[0, 0]).max() <= 2e-2, (an, cn, b, h)
                assert np.abs(f64(lse[b, h, :a_b]) - l[0, 0]).max() <= 4.5e-3, (an, cn, b, h)


def _sweep_shapes(n, seed):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        A = int(g.integers(65, 300))
        N = int(g.integers(A + 1, 1400))
        Nc = int(g.integers(1, N - A + 1))
        out.append((N, A, Nc, int(g.integers(0, 2)) * 3))
    return out


@pytest.mark.parametrize("N,A,Nc,n_skip", _sweep_shapes(12, 2024),
                         ids=lambda v: str(v))
def test_cached_workgroup_sweep(marca, N, A, Nc, n_skip):
    """Seeded random shapes through the workgroup path, with uniform and with
    per-sequence counts, the first two sequences against the oracle."""
    import oracle
    ts, active, cached = case(N, A, Nc, n_skip, seed=3 * N + A + Nc)
    B = ts[0].shape[0]
    lse = torch.empty((B, 2, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(*ts, cached, Nc=Nc, lse=lse)
    torch.cuda.synchronize()
    check_oracle(ts, cached, Nc, out, lse)

    g = np.random.default_rng(N + A)
    an = [int(g.integers(1, A + 1)), int(g.integers(1, A + 1))]
    cn = [int(g.integers(0, Nc + 1)), int(g.integers(0, Nc + 1))]
    a_len = torch.tensor(an, dtype=torch.int32, device=DEV).repeat(TILE)
    c_len = torch.tensor(cn, dtype=torch.int32, device=DEV).repeat(TILE)
    out = torch.full((B, 2, A, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    marca.mar_cache_attn_fwd_ragged(*ts, cached, a_len, c_len, out=out)
    torch.cuda.synchronize()
    q, ka, va, kc, vc = ts
    cl = cached.cpu().numpy()
    for b in range(2):
        assert (out[b, :, an[b]:].float() == 3.0).all()
        keep = cl[b, :cn[b]][(cl[b, :cn[b]] >= 0) & (cl[b, :cn[b]] < N)][None, :]
        for h in range(2):
            sl = lambda t, n=None: f64(t[b:b + 1, h:h + 1, :n])
            o, _ = oracle.cache_attention(sl(q, an[b]), sl(ka, an[b]), sl(va, an[b]), sl(kc), sl(vc),
                                          keep if keep.size else np.zeros((1, 1), np.int32),
                                          0.125, Nc=keep.shape[1])
            assert np.abs(f64(out[b, h, :an[b]]) - o[0, 0]).max() <= 2e-2, (b, h, an, cn)
