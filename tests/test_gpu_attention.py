"""GPU parity of mar_cache_attn_fwd against the CPU oracle.

Tolerances (from the accuracy targets of this path): fp32 -- normwise relative
error max|g - r| / max|r| <= 1e-5 per (sequence, head) tile; bf16 inputs with
float accumulation -- max-abs error <= 2e-2 on the unit-scale outputs.  The
log-sum-exp is compared to 1e-5 relative in fp32.  In bf16 the softmax
denominator sums the same bf16-rounded probabilities as the numerator, so it
carries a relative error of at most 2^-8 (the unit roundoff of bf16's 8-bit
significand) plus float accumulation (at most T * 2^-24 for T keys, below
5e-4 up to 8192 keys): the log-sum-exp bound is ln(1 + 2^-8) + 5e-4 < 4.5e-3
absolute.  A nearly one-hot softmax comes close to it: its one dominant
probability carries the whole rounding error.
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


def np64(t):
    return t.detach().double().cpu().numpy()


def oracle_units(x, units, Nc):
    """Oracle output/lse for the listed (b, h) units of an attention_inputs dict."""
    import oracle
    cfg = x["cfg"]
    outs, lses = [], []
    cached = x["cached"].cpu().numpy()
    for b, h in units:
        sl = lambda k: np64(x[k][b:b + 1, h:h + 1])
        o, l = oracle.cache_attention(sl("q_a"), sl("k_a"), sl("v_a"), sl("k_cache"), sl("v_cache"),
                                      cached[b:b + 1], cfg.D ** -0.5, Nc=Nc)
        outs.append(o[0, 0])
        lses.append(l[0, 0])
    return np.stack(outs), np.stack(lses)


def torch_f32_all_units(x, Nc):
    """Every unit's attention over [active rows ; cached rows] in float32 torch
    operations on the device: the oracle's definition, for all units at once
    (an any-size check beside the oracle's sampled units)."""
    q = x["q_a"].float()
    B, H, A, D = q.shape
    gi = x["cached"][:, :Nc].long()[:, None, :, None].expand(B, H, Nc, D)
    k = torch.cat([x["k_a"].float(), torch.gather(x["k_cache"].float(), 2, gi)], 2)
    v = torch.cat([x["v_a"].float(), torch.gather(x["v_cache"].float(), 2, gi)], 2)
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * D ** -0.5
    return torch.matmul(torch.softmax(s, -1), v)


def check(got_out, got_lse, ref_out, ref_lse, dtype):
    if dtype == "f32":
        for u in range(ref_out.shape[0]):
            err = np.abs(got_out[u] - ref_out[u]).max() / np.abs(ref_out[u]).max()
            assert err <= 1e-5, f"unit {u}: normwise error {err}"
        np.testing.assert_allclose(got_lse, ref_lse, rtol=1e-5, atol=1e-6)
    else:
        err = np.abs(got_out - ref_out).max()
        assert err <= 2e-2, f"max-abs error {err}"
        assert np.abs(got_lse - ref_lse).max() <= 4.5e-3


def run(marca, x, Nc=None, cached=None):
    cfg = x["cfg"]
    B, H, A, D = x["q_a"].shape
    lse = torch.empty((B, H, A), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                   x["cached"] if cached is None else cached, Nc=Nc, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def small_cfg(dtype, B, H, N, A, stale=True, n_prefix=0, seed=77):
    return Config("t", B=B, H=H, D=64, N=N, n_prefix=n_prefix, A=A, n_gen=0, n_prev=0, K=0,
                  layers=1, dtype=dtype, stale=stale, seed=seed)


def test_tiny_exact_equivalence(marca):
    """Tiny fp32 case with a current cache: equals full attention over all N tokens."""
    import oracle
    cfg = CONFIGS["tiny"]
    x = attention_inputs(cfg, DEV)
    out, lse = run(marca, x)
    ref_o, ref_l = oracle_units(x, [(0, 0), (0, 1)], cfg.Nc)
    check(np64(out)[0], np64(lse)[0], ref_o, ref_l, "f32")
    # and the oracle's result is full attention of the active queries over all N tokens
    q = np64(x["q_a"])
    kc, vc = np64(x["k_cache"]), np64(x["v_cache"])
    full = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(kc), torch.from_numpy(vc), scale=cfg.D ** -0.5)
    err = np.abs(np64(out) - full.numpy()).max() / np.abs(full.numpy()).max()
    assert err <= 1e-5


@pytest.mark.parametrize("A,Nc", [(16, 0), (16, 48), (17, 31), (24, 296), (33, 1), (48, 272),
                                  (64, 256), (65, 100), (100, 37), (128, 960 - 800)])
def test_bf16_mfma_path_ragged(marca, A, Nc):
    cfg = small_cfg("bf16", B=2, H=3, N=A + Nc + 5, A=A, seed=A * 1000 + Nc)
    x = attention_inputs(cfg, DEV, ascending=False)
    out, lse = run(marca, x, Nc=Nc, cached=x["cached"][:, :Nc].contiguous())
    units = [(b, h) for b in range(2) for h in range(3)]
    ref_o, ref_l = oracle_units({**x, "cached": x["cached"][:, :max(Nc, 1)]}, units, Nc)
    got_o = np64(out).reshape(6, A, 64)
    got_l = np64(lse).reshape(6, A)
    check(got_o, got_l, ref_o, ref_l, "bf16")


@pytest.mark.parametrize("dtype,A", [("bf16", 1), ("bf16", 5), ("bf16", 15), ("f32", 1),
                                     ("f32", 8), ("f32", 33), ("f32", 70)])
def test_vector_and_fp32_paths(marca, dtype, A):
    """Below 16 active queries (bf16 and fp32) the per-unit vector kernel runs;
    fp32 with 16 or more the fp32 matrix-core kernel (one and two query groups)."""
    Nc = 150
    cfg = small_cfg(dtype, B=2, H=2, N=A + Nc, A=A, seed=500 + A)
    x = attention_inputs(cfg, DEV, ascending=False)
    out, lse = run(marca, x)
    units = [(b, h) for b in range(2) for h in range(2)]
    ref_o, ref_l = oracle_units(x, units, Nc)
    check(np64(out).reshape(4, A, 64), np64(lse).reshape(4, A), ref_o, ref_l, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_list_and_invalid_entries_are_skipped(marca, dtype):
    """ldc > Nc, -1 padding, and an out-of-range entry behave as if absent."""
    import oracle
    A, N = 24, 200
    cfg = small_cfg(dtype, B=2, H=2, N=N, A=A, seed=31)
    x = attention_inputs(cfg, DEV)
    cached = x["cached"].cpu().numpy()  # [B, 176] ascending
    Nc = cached.shape[1]
    padded = np.full((2, N), -1, np.int32)
    padded[:, :Nc] = cached
    bad = padded.copy()
    bad[:, 5] = N + 3          # out of range -> skipped
    bad[:, 9] = -7
    got_pad, _ = run(marca, x, Nc=Nc, cached=torch.from_numpy(padded).to(DEV))
    got_bad, _ = run(marca, x, Nc=Nc, cached=torch.from_numpy(bad).to(DEV))
    keep = np.delete(cached, [5, 9], axis=1)
    ref_pad, _ = oracle_units({**x, "cached": torch.from_numpy(cached)}, [(1, 1)], Nc)
    ref_bad, _ = oracle_units({**x, "cached": torch.from_numpy(keep)}, [(1, 1)], Nc - 2)
    tol = 1e-5 if dtype == "f32" else 2e-2
    scale_p = np.abs(ref_pad).max() if dtype == "f32" else 1.0
    assert np.abs(np64(got_pad)[1, 1] - ref_pad[0]).max() <= tol * scale_p
    assert np.abs(np64(got_bad)[1, 1] - ref_bad[0]).max() <= tol * scale_p


def test_full_attention_case_and_single_query(marca):
    """A == N, Nc == 0 (the full-attention layers) and A == 1."""
    for dtype, A in (("bf16", 64), ("f32", 64), ("bf16", 1)):
        N = A if A > 1 else 40
        Nc = 0 if A == N else N - A
        cfg = small_cfg(dtype, B=1, H=2, N=N, A=A, stale=False, seed=9 + A)
        x = attention_inputs(cfg, DEV)
        out, lse = run(marca, x, Nc=Nc, cached=None if Nc == 0 else x["cached"])
        ref_o, ref_l = oracle_units({**x, "cached": torch.zeros((1, 1), dtype=torch.int32)}
                                    if Nc == 0 else x, [(0, 0), (0, 1)], Nc)
        check(np64(out)[0], np64(lse)[0], ref_o, ref_l, dtype)


@pytest.mark.parametrize("A,Nc", [(40, 200), (24, 296), (100, 150)])
def test_batch_of_256_units(marca, A, Nc):
    """256 (sequence, head) units, including more queries than one wave takes."""
    cfg = small_cfg("bf16", B=32, H=8, N=A + Nc, A=A, seed=60 + A)
    x = attention_inputs(cfg, DEV)
    out, lse = run(marca, x)
    units = [(0, 0), (31, 7), (17, 3), (5, 6)]
    ref_o, ref_l = oracle_units(x, units, Nc)
    check(np.stack([np64(out[b, h]) for b, h in units]),
          np.stack([np64(lse[b, h]) for b, h in units]), ref_o, ref_l, "bf16")
    # the fused update must also write each unit's active rows exactly once
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    act = x["active"].to(torch.int32).contiguous()
    out2 = marca.mar_cache_attn_fwd_update(x["q_a"], x["k_a"], x["v_a"], kc, vc, x["cached"], act)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)
    ak = act.long()[:, None, :, None].expand(-1, 8, -1, 64)
    assert torch.equal(torch.gather(kc, 2, ak), x["k_a"])
    assert torch.equal(torch.gather(vc, 2, ak), x["v_a"])


@pytest.mark.parametrize("N", [128, 129, 200, 320])
def test_full_attention_layers(marca, N):
    """A == N, Nc == 0 with many queries: the workgroup kernel that shares each
    unit's K/V across its query blocks (ragged last block and last chunk)."""
    cfg = small_cfg("bf16", B=2, H=3, N=N, A=N, stale=False, seed=40 + N)
    x = attention_inputs(cfg, DEV)
    out, lse = run(marca, x, Nc=0, cached=None)
    units = [(0, 0), (1, 2), (0, 1)]
    ref_o, ref_l = oracle_units({**x, "cached": torch.zeros((1, 1), dtype=torch.int32)}, units, 0)
    got_o = np.stack([np64(out[b, h]) for b, h in units])
    got_l = np.stack([np64(lse[b, h]) for b, h in units])
    check(got_o, got_l, ref_o, ref_l, "bf16")


def test_full_attention_mar_l_layer(marca):
    """A full-attention layer at the MAR-L shape (128 sequences, 16 heads, N = 320)."""
    from mar_workloads import device_normal
    B, H, N = 128, 16, 320
    q = device_normal((B, H, N, 64), 301, DEV, torch.bfloat16)
    k = device_normal((B, H, N, 64), 302, DEV, torch.bfloat16)
    v = device_normal((B, H, N, 64), 303, DEV, torch.bfloat16)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    out = marca.mar_cache_attn_fwd(q, k, v, k, v, None, Nc=0, lse=lse)
    torch.cuda.synchronize()
    import oracle
    for b, h in ((0, 0), (127, 15), (64, 7)):
        sl = lambda t: np64(t[b:b + 1, h:h + 1])
        o, l = oracle.cache_attention(sl(q), sl(k), sl(v), sl(k), sl(v),
                                      np.zeros((1, 1), np.int32), 0.125, Nc=0)
        check(np64(out[b, h])[None], np64(lse[b, h])[None], o[0], l[0], "bf16")


@pytest.mark.parametrize("name,update", [("mar_h", False), ("highres", False),
                                         ("highres", True)])
def test_full_attention_full_size(marca, name, update):
    """Full-attention layers at the MAR-H shape (256 sequences, 20 heads,
    N = 320) and the high-res shape (N = 1088: four workgroups per unit, the
    last with idle waves); with the update, a refresh step's layer, whose
    caches must come out equal to the fresh K/V."""
    from mar_workloads import device_normal
    import oracle
    cfg = CONFIGS[name]
    B, H, N = cfg.B, cfg.H, cfg.N
    q, k, v = (device_normal((B, H, N, 64), 310 + i, DEV, torch.bfloat16) for i in range(3))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    if update:
        kc, vc = torch.zeros_like(k), torch.zeros_like(v)
        out = marca.mar_cache_attn_fwd_update(q, k, v, kc, vc, None, None, Nc=0, lse=lse)
    else:
        out = marca.mar_cache_attn_fwd(q, k, v, k, v, None, Nc=0, lse=lse)
    torch.cuda.synchronize()
    if update:
        assert torch.equal(kc, k) and torch.equal(vc, v)
        del kc, vc
    rng = np.random.default_rng(cfg.seed + 1)
    units = [(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))]
    for b, h in units:
        sl = lambda t: np64(t[b:b + 1, h:h + 1])
        o, l = oracle.cache_attention(sl(q), sl(k), sl(v), sl(k), sl(v),
                                      np.zeros((1, 1), np.int32), 0.125, Nc=0)
        check(np64(out[b, h])[None], np64(lse[b, h])[None], o[0], l[0], "bf16")


@pytest.mark.parametrize("B,H,N,update", [(64, 20, 200, False), (64, 20, 200, True),
                                          (16, 40, 650, False), (16, 40, 650, True)])
def test_full_attention_several_items_per_workgroup(marca, B, H, N, update):
    """More (unit, query block) items than resident workgroups, so each
    workgroup carries its chunk stream and its prefetched queries from one
    item to the next: an odd number of chunks per unit (the LDS buffer of an
    item's first chunk alternates), and with N = 650 three blocks per unit and
    a partial last chunk.  With the update the caches must come out equal to
    the fresh K/V."""
    from mar_workloads import device_normal
    import oracle
    q, k, v = (device_normal((B, H, N, 64), 900 + N + i, DEV, torch.bfloat16) for i in range(3))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    if update:
        kc, vc = torch.zeros_like(k), torch.zeros_like(v)
        out = marca.mar_cache_attn_fwd_update(q, k, v, kc, vc, None, None, Nc=0, lse=lse)
    else:
        out = marca.mar_cache_attn_fwd(q, k, v, k, v, None, Nc=0, lse=lse)
    torch.cuda.synchronize()
    if update:
        assert torch.equal(kc, k) and torch.equal(vc, v)
        del kc, vc
    rng = np.random.default_rng(N + update)
    units = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(B)), int(rng.integers(H)))
                                        for _ in range(4)]
    for b, h in units:
        sl = lambda t: np64(t[b:b + 1, h:h + 1])
        o, l = oracle.cache_attention(sl(q), sl(k), sl(v), sl(k), sl(v),
                                      np.zeros((1, 1), np.int32), 0.125, Nc=0)
        check(np64(out[b, h])[None], np64(lse[b, h])[None], o[0], l[0], "bf16")
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("name", ["mar_b", "mar_l", "mar_h", "highres"])
def test_full_size_sampled_units(marca, name):
    """Full-size MAR shapes, the launch configuration the benchmark times;
    the oracle checks the first and last (b,h) units and six seeded ones, and
    a float32 torch computation of the same definition checks every unit."""
    cfg = CONFIGS[name]
    x = attention_inputs(cfg, DEV)
    out, lse = run(marca, x)
    rng = np.random.default_rng(cfg.seed)
    units = [(0, 0), (cfg.B - 1, cfg.H - 1)] + [
        (int(rng.integers(cfg.B)), int(rng.integers(cfg.H))) for _ in range(6)]
    ref_o, ref_l = oracle_units(x, units, cfg.Nc)
    got_o = np.stack([np64(out[b, h]) for b, h in units])
    got_l = np.stack([np64(lse[b, h]) for b, h in units])
    check(got_o, got_l, ref_o, ref_l, "bf16")
    # any-size property: every output is a convex combination of value rows
    vmax = max(float(x["v_a"].float().abs().max()), float(x["v_cache"].float().abs().max()))
    assert float(out.float().abs().max()) <= vmax * (1 + 2 ** -6)
    assert torch.isfinite(out.float()).all()
    # every unit against the same definition in float32 torch operations
    ref_all = torch_f32_all_units(x, cfg.Nc)
    assert float((out.float() - ref_all).abs().max()) <= 2e-2
    del ref_all


def test_deterministic(marca):
    cfg = CONFIGS["mar_b"]
    x = attention_inputs(cfg, DEV)
    o1, l1 = run(marca, x)
    o2, l2 = run(marca, x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_cached_order_invariance(marca):
    cfg = small_cfg("bf16", B=2, H=2, N=300, A=48, seed=4)
    x = attention_inputs(cfg, DEV, ascending=True)
    o1, _ = run(marca, x)
    perm = torch.stack([row[torch.randperm(row.numel(), generator=torch.Generator().manual_seed(1))
                             .to(DEV)] for row in x["cached"]]).contiguous()
    o2, _ = run(marca, x, cached=perm)
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
