"""GPU parity of the few-unit attention path: with few (sequence, head) units
the library runs several waves per unit, each over its own contiguous range of
the unit's 32-row chunks, and merges their partial (max, sum, weighted sum)
states before the output is written.  With many units every unit runs on one
wave.

Each case runs the same two sequences twice: alone (2 sequences x 2 heads, so
the unit is split over waves) and tiled into a batch of 160 sequences (320
units: one wave per unit).  Both results are checked against the oracle
(bf16: max-abs 2e-2, log-sum-exp 4.5e-3), and against each other.  The
kernel rounds the softmax probabilities to bf16 (relative error at most 2^-8)
relative to each wave's own running maximum, so the two schedules round them
differently; the denominator sums the same rounded values, so each output
element is within 2^-7 * sum_i w_i |v_i| of the exact one (w: the softmax
weights), and the two differ by at most 2^-6 * sum_i w_i |v_i| plus one bf16
unit in the last place of the output.  sum_i w_i |v_i| is the oracle's
attention with |V| as the values.

The chunk counts are chosen to leave waves without chunks: 9 chunks over 4
waves (ranges of 3: the fourth wave is empty) and 17 chunks over 8 waves
(ranges of 3: the last two are empty); per-sequence counts leave still more.
"""
import numpy as np
import pytest
import torch

from mar_workloads import device_normal

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
TILE = 80  # copies of the two sequences in the one-wave batch (2 * 80 * H=2 = 320 units)

# (N, A, Nc): tokens, active queries, cached entries
CASES = [(300, 40, 230),    # 9 chunks, split 4: an empty wave
         (540, 20, 500),    # 17 chunks, split 8: two empty waves
         (320, 48, 272),    # the MAR-L layer shape: 10 chunks, split 4
         (1088, 128, 960),  # two query groups of 64, 34 chunks, split 4
         (700, 16, 600)]    # a single query tile


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


def pair(N, A, Nc, seed):
    """Two sequences x two heads: Q/K/V of the active rows, stale caches, the
    active positions and the cached list (distinct tokens per sequence)."""
    B, H = 2, 2
    q, ka, va = (device_normal((B, H, A, 64), seed + i, DEV, torch.bfloat16) for i in range(3))
    kc, vc = (device_normal((B, H, N, 64), seed + 3 + i, DEV, torch.bfloat16) for i in range(2))
    g = torch.Generator().manual_seed(seed)
    perms = [torch.randperm(N, generator=g) for _ in range(B)]
    active = torch.stack([p[:A] for p in perms]).to(torch.int32).to(DEV)
    cached = torch.stack([p[A:A + Nc] for p in perms]).to(torch.int32).to(DEV)
    return [q, ka, va, kc, vc], active, cached


def tiled(ts):
    return [t.repeat(TILE, *([1] * (t.dim() - 1))).contiguous() for t in ts]


def oracle_check(ts, cached, out, lse, an=None, cn=None):
    """Checks out/lse against the oracle on the 4 units; returns the bound on
    the difference of two schedules per output element (zero past a count)."""
    import oracle
    q, ka, va, kc, vc = ts
    cl = cached.cpu().numpy()
    bound = np.zeros(tuple(out.shape))
    for b in range(2):
        a_b = q.shape[2] if an is None else int(an[b])
        c_b = cl.shape[1] if cn is None else int(cn[b])
        if a_b == 0:
            continue
        for h in range(2):
            sl = lambda t, n: f64(t[b:b + 1, h:h + 1, :n])
            args = (sl(q, a_b), sl(ka, a_b), sl(va, a_b), f64(kc[b:b + 1, h:h + 1]),
                    f64(vc[b:b + 1, h:h + 1]))
            o, l = oracle.cache_attention(*args, cl[b:b + 1, :max(c_b, 1)], 0.125, Nc=c_b)
            err = np.abs(f64(out[b, h, :a_b]) - o[0, 0]).max()
            assert err <= 2e-2, f"unit ({b},{h}): max-abs {err}"
            if lse is not None:
                assert np.abs(f64(lse[b, h, :a_b]) - l[0, 0]).max() <= 4.5e-3, (b, h)
            wabs, _ = oracle.cache_attention(args[0], args[1], np.abs(args[2]), args[3],
                                             np.abs(args[4]), cl[b:b + 1, :max(c_b, 1)], 0.125,
                                             Nc=c_b)
            bound[b, h, :a_b] = 2.0 ** -6 * wabs[0, 0]
    return bound


def close_schedules(a, b, bound):
    """Two schedules' bf16 outputs: within bound plus one ulp of the larger."""
    a, b = f64(a), f64(b)
    m = np.maximum(np.abs(a), np.abs(b))
    ulp = np.exp2(np.floor(np.log2(np.maximum(m, 1e-30))) - 7)
    excess = np.abs(a - b) - (bound + ulp)
    assert (excess <= 0).all(), (np.abs(a - b).max(), excess.max())


@pytest.mark.parametrize("N,A,Nc", CASES)
def test_split_matches_one_wave_and_oracle(marca, N, A, Nc):
    ts, active, cached = pair(N, A, Nc, seed=31 * N + A)
    lse = torch.empty((2, 2, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(*ts, cached, Nc=Nc, lse=lse)
    big = tiled(ts)
    big_lse = torch.empty((2 * TILE, 2, A), dtype=torch.float32, device=DEV)
    big_out = marca.mar_cache_attn_fwd(*big, cached.repeat(TILE, 1).contiguous(), Nc=Nc,
                                       lse=big_lse)
    torch.cuda.synchronize()
    bound = oracle_check(ts, cached, out, lse)
    oracle_check(ts, cached, big_out[:2], big_lse[:2])
    for t in range(TILE):  # every copy in the big batch computes the same thing
        assert torch.equal(big_out[2 * t:2 * t + 2], big_out[:2])
    close_schedules(out, big_out[:2], bound)
    # each log-sum-exp is within 4.5e-3 of the exact one
    np.testing.assert_allclose(f64(lse), f64(big_lse[:2]), rtol=0, atol=9e-3)


@pytest.mark.parametrize("N,A,Nc", [CASES[0], CASES[1], CASES[3]])
def test_split_fused_update(marca, N, A, Nc):
    """The fused cache update under the split: the same output bits as the
    split attention, and every active row written exactly once."""
    import oracle
    ts, active, cached = pair(N, A, Nc, seed=17 * N + A)
    q, ka, va, kc, vc = ts
    out = marca.mar_cache_attn_fwd(*ts, cached, Nc=Nc)
    kc2, vc2 = kc.clone(), vc.clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out2 = marca.mar_cache_attn_fwd_update(q, ka, va, kc2, vc2, cached, active, Nc=Nc,
                                           err_count=err)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    assert int(err.item()) == 0
    kr, vr, skipped = oracle.kv_scatter(raw(kc), raw(vc), raw(ka), raw(va), active.cpu().numpy())
    assert skipped == 0
    assert np.array_equal(raw(kc2), kr) and np.array_equal(raw(vc2), vr)


@pytest.mark.parametrize("N,A,Nc", [CASES[0], CASES[1], CASES[3]])
def test_split_ragged(marca, N, A, Nc):
    """Per-sequence counts: short sequences leave most waves of their unit
    without chunks; a sequence with no active queries writes nothing."""
    ts, active, cached = pair(N, A, Nc, seed=13 * N + A)
    for an, cn in [(A, Nc), (1, 0), (0, Nc), (A // 2 + 1, 7), (A - 1, Nc - 33)]:
        a_len = torch.tensor([an, A], dtype=torch.int32, device=DEV)
        c_len = torch.tensor([cn, Nc // 2], dtype=torch.int32, device=DEV)
        out = torch.full((2, 2, A, 64), 3.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.full((2, 2, A), 7.0, dtype=torch.float32, device=DEV)
        marca.mar_cache_attn_fwd_ragged(*ts, cached, a_len, c_len, out=out, lse=lse)
        big_out = marca.mar_cache_attn_fwd_ragged(*tiled(ts), cached.repeat(TILE, 1).contiguous(),
                                                  a_len.repeat(TILE), c_len.repeat(TILE))
        torch.cuda.synchronize()
        assert (out[0, :, an:].float() == 3.0).all() and (lse[0, :, an:] == 7.0).all()
        bound = oracle_check(ts, cached, out, lse, an=[an, A], cn=[cn, Nc // 2])
        close_schedules(out[0, :, :an], big_out[0, :, :an], bound[0, :, :an])
        close_schedules(out[1], big_out[1], bound[1])
