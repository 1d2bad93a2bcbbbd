"""GPU parity of the KV scatter / full refresh, refresh top-K, cosine gate and
CFG residual kernels against the CPU oracle.

Integer outputs are compared bit for bit.  Where a float decides an integer
(top-K ranking, gate threshold) the oracle takes the decision on the GPU's own
floats (bit-exact comparison), and against the oracle's own floats only away
from the decision boundary.  Float outputs: refresh scores within normwise
relative 1e-5; cosines within 1e-5 absolute (both sides reduce the same values);
CFG residual and reused uncond bit-exact; the guidance mix within one float32
rounding of the exact value.
"""
import numpy as np
import pytest
import torch

import oracle
from mar_workloads import (CONFIGS, attention_inputs, cfg_outputs, device_gate_features,
                           device_normal, gate_features, generation_order)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


@pytest.fixture(scope="module")
def marca():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cache_aware_attention_amd as m
    return m


def bits(t):
    return t.view(torch.int16).cpu().numpy() if t.element_size() == 2 else \
        t.view(torch.int32).cpu().numpy()


# ---------------------------------------------------------------- scatter --

@pytest.mark.parametrize("name", ["tiny", "mar_b", "mar_l"])
def test_scatter_partial_bit_exact(marca, name):
    cfg = CONFIGS[name]
    x = attention_inputs(cfg, DEV)
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    marca.mar_kv_scatter_refresh(kc, vc, x["k_a"], x["v_a"], x["active"], err_count=err)
    torch.cuda.synchronize()
    rk, rv, sk = oracle.kv_scatter(bits(x["k_cache"]), bits(x["v_cache"]), bits(x["k_a"]),
                                   bits(x["v_a"]), x["active"].cpu().numpy())
    assert (bits(kc) == rk).all() and (bits(vc) == rv).all()
    assert int(err.item()) == sk == 0


def test_scatter_skips_and_counts_invalid(marca):
    cfg = CONFIGS["mar_b"]
    x = attention_inputs(cfg, DEV)
    idx = x["active"].clone()
    idx[0, 3] = -1
    idx[5, 0] = cfg.N
    idx[7, cfg.A - 1] = 10 ** 6
    # a padded index buffer (ld_idx > M) as written by the top-K kernel
    wide = torch.full((cfg.B, cfg.A + 7), -1, dtype=torch.int32, device=DEV)
    wide[:, :cfg.A] = idx
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    marca.mar_kv_scatter_refresh(kc, vc, x["k_a"], x["v_a"], wide, err_count=err)
    torch.cuda.synchronize()
    rk, rv, sk = oracle.kv_scatter(bits(x["k_cache"]), bits(x["v_cache"]), bits(x["k_a"]),
                                   bits(x["v_a"]), idx.cpu().numpy())
    assert (bits(kc) == rk).all() and (bits(vc) == rv).all()
    assert int(err.item()) == sk == 3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_full_refresh_copies(marca, dtype):
    B, H, N, D = 3, 5, 77, 64
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = device_normal((B, H, N, D), 1, DEV, dt)
    vc = device_normal((B, H, N, D), 2, DEV, dt)
    kn = device_normal((B, H, N, D), 3, DEV, dt)
    vn = device_normal((B, H, N, D), 4, DEV, dt)
    marca.mar_kv_scatter_refresh(kc, vc, kn, vn, None)
    torch.cuda.synchronize()
    assert torch.equal(kc, kn) and torch.equal(vc, vn)


# ---------------------------------------------------------------- top-K ----

def topk_case(marca, B, H, G, N, n_gp, K, dtype="bf16", seed=0, dup=False):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = device_normal((B, H, G, 64), seed * 10 + 1, DEV, dt)
    k = device_normal((B, H, N, 64), seed * 10 + 2, DEV, dt)
    if dup:  # identical key rows => identical scores; the lower index must win
        k[:, :, N - 1] = k[:, :, 1]
        k[:, :, N - 2] = k[:, :, 2]
    g = torch.Generator().manual_seed(seed)
    gp = torch.stack([torch.randperm(N, generator=g)[:n_gp] for _ in range(B)]).to(
        dtype=torch.int32, device=DEV)
    scores, act, cac, clen = marca.mar_refresh_topk(q, k, gp, n_gp, K)
    torch.cuda.synchronize()
    return q, k, gp, scores, act, cac, clen


def check_topk(q, k, gp, scores, act, cac, clen, K):
    D = q.shape[-1]
    s_gpu = scores.double().cpu().numpy()
    s_ref = oracle.refresh_scores(q.double().cpu().numpy(), k.double().cpu().numpy(), D ** -0.5)
    err = np.abs(s_gpu - s_ref).max() / np.abs(s_ref).max()
    assert err <= 1e-5, f"scores normwise error {err}"
    # bit-exact selection on the GPU's own scores
    ra, rc, rl = oracle.refresh_select(s_gpu, gp.cpu().numpy(), K, ld_cached=cac.shape[1])
    assert (act.cpu().numpy()[:, :ra.shape[1]] == ra).all()
    assert (cac.cpu().numpy() == rc).all()
    assert (clen.cpu().numpy() == rl).all()
    # against the oracle's own scores where the K-th / (K+1)-th gap is clear
    oa, _, _ = oracle.refresh_select(s_ref, gp.cpu().numpy(), K)
    n_gp = gp.shape[1]
    for b in range(s_ref.shape[0]):
        elig = np.setdiff1d(np.arange(s_ref.shape[1]), gp[b].cpu().numpy())
        srt = np.sort(s_ref[b, elig])[::-1]
        if K < srt.size and K > 0:
            gap = srt[K - 1] - srt[K]
            if gap > 1e-4 * srt[K - 1]:
                assert set(oa[b, n_gp:]) == set(act[b, n_gp:n_gp + K].cpu().numpy())


@pytest.mark.parametrize("B,H,G,N,n_gp,K,dtype", [
    (3, 2, 5, 70, 9, 7, "bf16"), (2, 3, 1, 33, 0, 4, "f32"), (2, 2, 16, 320, 32, 16, "bf16"),
    (2, 2, 17, 100, 20, 30, "bf16"), (1, 4, 40, 257, 60, 40, "f32"), (2, 1, 3, 64, 10, 0, "bf16"),
    (2, 2, 26, 1088, 52, 76, "bf16"), (1, 2, 64, 200, 10, 20, "bf16"),
    (1, 2, 64, 300, 10, 20, "bf16"),
    # the register-resident scores take up to 16 queries and 320 keys; the
    # selection keeps up to 2048 keys in registers (one round of one token per
    # thread up to 1024, two rounds up to 2048), past that it reads LDS
    (2, 2, 16, 319, 32, 16, "bf16"), (2, 2, 16, 321, 32, 16, "bf16"),
    (2, 2, 16, 500, 40, 25, "bf16"), (2, 2, 12, 700, 30, 40, "bf16"),
    (1, 2, 16, 1024, 20, 30, "bf16"), (1, 2, 16, 1025, 20, 30, "bf16"),
    (1, 2, 16, 1500, 40, 30, "bf16"), (1, 2, 16, 2048, 40, 30, "bf16"),
    (1, 2, 16, 2500, 40, 30, "bf16"),
    # one token (every other key of the only tile masked; its score is 1) and one
    # token past a whole tile
    (1, 2, 4, 1, 0, 1, "bf16"), (2, 2, 16, 17, 0, 5, "bf16")])
def test_topk_small(marca, B, H, G, N, n_gp, K, dtype):
    out = topk_case(marca, B, H, G, N, n_gp, K, dtype, seed=B * 100 + N)
    check_topk(*out, K)


def test_topk_ties_lower_index(marca):
    q, k, gp, scores, act, cac, clen = topk_case(marca, 2, 2, 4, 50, 0, 49, dup=True, seed=3)
    s = scores.cpu().numpy()
    assert (s[:, 1] == s[:, 49]).all() and (s[:, 2] == s[:, 48]).all()
    check_topk(q, k, gp, scores, act, cac, clen, 49)
    a = act.cpu().numpy()
    for b in range(2):
        pos = {int(j): r for r, j in enumerate(a[b])}
        assert pos[1] < pos[49] and pos[2] < pos[48]


def test_topk_repeated_gp_entries(marca):
    """Repeated G/P entries exclude a token once; the cached set grows accordingly."""
    B, H, G, N = 2, 2, 3, 20
    q = device_normal((B, H, G, 64), 5, DEV, torch.bfloat16)
    k = device_normal((B, H, N, 64), 6, DEV, torch.bfloat16)
    gp = torch.tensor([list(range(15)) + [0, 1], list(range(5, 20)) + [5, 5]], dtype=torch.int32,
                      device=DEV)
    scores, act, cac, clen = marca.mar_refresh_topk(q, k, gp, 17, 3)
    torch.cuda.synchronize()
    check_topk(q, k, gp, scores, act, cac, clen, 3)
    assert clen.cpu().numpy().tolist() == [20 - 15 - 3, 20 - 15 - 3]
    assert (act[:, 17:].cpu().numpy() >= 0).all()


def test_topk_full_size_mar_l(marca):
    """MAR-L: 128 sequences, 16 heads, 16 generating queries, N 320, |G|+|P| = 32, K 16;
    G/P taken straight from the generation order (a strided view)."""
    cfg = CONFIGS["mar_l"]
    order = torch.from_numpy(generation_order(cfg)).to(DEV)
    gp = order[:, 100:132]  # previous 16 then current 16 of some step
    q = device_normal((cfg.B, cfg.H, 16, 64), 11, DEV, torch.bfloat16)
    k = device_normal((cfg.B, cfg.H, cfg.N, 64), 12, DEV, torch.bfloat16)
    scores, act, cac, clen = marca.mar_refresh_topk(q, k, gp, 32, 16)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 127]
    check_topk(q[rows], k[rows], gp[rows].contiguous(), scores[rows], act[rows], cac[rows],
               clen[rows], 16)
    # any-size properties: scores sum to 1; partition covers every token once
    assert torch.allclose(scores.sum(1), torch.ones(cfg.B, device=DEV), atol=1e-4)
    a = act.cpu().numpy()
    c = cac.cpu().numpy()
    L = clen.cpu().numpy()
    for b in range(cfg.B):
        allv = np.concatenate([a[b], c[b, :L[b]]])
        assert sorted(allv.tolist()) == list(range(cfg.N))
        assert (np.diff(c[b, :L[b]]) > 0).all()


def test_topk_full_size_highres(marca):
    """High-res: 64 sequences, 16 heads, 26 generating queries, N 1088, |G|+|P| =
    52, K 76 (a budget of 128), as the high-res decode's layer 2 calls it:
    sampled sequences against the oracle, properties on all of them."""
    cfg = CONFIGS["highres"]
    order = torch.from_numpy(generation_order(cfg)).to(DEV)
    gp = order[:, 300:352]
    q = device_normal((cfg.B, cfg.H, 26, 64), 13, DEV, torch.bfloat16)
    k = device_normal((cfg.B, cfg.H, cfg.N, 64), 14, DEV, torch.bfloat16)
    scores, act, cac, clen = marca.mar_refresh_topk(q, k, gp, 52, 76)
    torch.cuda.synchronize()
    rows = [0, 21, 42, 63]
    check_topk(q[rows], k[rows], gp[rows].contiguous(), scores[rows], act[rows], cac[rows],
               clen[rows], 76)
    assert torch.allclose(scores.sum(1), torch.ones(cfg.B, device=DEV), atol=1e-4)
    a = act.cpu().numpy()
    c = cac.cpu().numpy()
    L = clen.cpu().numpy()
    for b in range(cfg.B):
        allv = np.concatenate([a[b], c[b, :L[b]]])
        assert sorted(allv.tolist()) == list(range(cfg.N))
        assert (np.diff(c[b, :L[b]]) > 0).all()


# ---------------------------------------------------------------- gate -----

# Both sides reduce the same input values (a bf16 product is exact in fp32):
# the kernel sums in fp32 along chains of at most W/64 + 6 additions per
# quantity (elements per lane, then the lane tree), so each of <x,y>, |x|^2 and
# |y|^2 carries an error of at most (W/64 + 6) 2^-24 of its sum of magnitudes;
# by Cauchy-Schwarz the cosine then moves by at most about twice that plus the
# roundings of the square roots and the division: under 6e-6 for W <= 2048
# (under 1e-5 up to W = 4096).  A dropped 16-byte piece moves it by ~1e-3.
GATE_COS_TOL = 1e-5


def reuse_lists(mask):
    """The ascending positions with reuse 1 of each row, -1 padded, and their
    counts: the definition of the gate's optional reuse list, from a mask."""
    B, N = mask.shape
    idx = np.full((B, N), -1, np.int32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        pos = np.flatnonzero(mask[b])
        idx[b, :len(pos)] = pos
        cnt[b] = len(pos)
    return idx, cnt


def gate_with_reuse(marca, x, y, tau=0.95):
    B, N = x.shape[0], x.shape[1]
    ridx = torch.full((B, N), 7, dtype=torch.int32, device=DEV)  # stale values must be overwritten
    rlen = torch.full((B,), 7, dtype=torch.int32, device=DEV)
    cos, reuse, cidx, clen = marca.mar_cos_gate(x, y, tau, reuse_idx=ridx, reuse_len=rlen)
    return cos, reuse, cidx, clen, ridx, rlen

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_small_bit_exact(marca, dtype):
    x, y, rho = gate_features(3, 100, 256, seed=21, device=DEV, dtype=dtype)
    cos, reuse, cidx, clen, ridx, rlen = gate_with_reuse(marca, x, y)
    torch.cuda.synchronize()
    c_gpu = cos.double().cpu().numpy()
    tau32 = float(np.float32(0.95))
    r2, c2, l2 = oracle.gate_from_cos(c_gpu, tau32)
    assert (reuse.cpu().numpy() == r2).all() and (cidx.cpu().numpy() == c2).all()
    assert (clen.cpu().numpy() == l2).all()
    ri, rl = reuse_lists(r2)
    assert (ridx.cpu().numpy() == ri).all() and (rlen.cpu().numpy() == rl).all()
    assert (rl + l2 == 100).all()
    c_ref, r_ref, _, _ = oracle.cos_gate(x.double().cpu().numpy(), y.double().cpu().numpy(), tau32)
    assert np.abs(c_gpu - c_ref).max() <= GATE_COS_TOL
    away = np.abs(c_ref - tau32) > 1e-4
    assert (reuse.cpu().numpy()[away] == r_ref[away]).all()


@pytest.mark.parametrize("dtype,B,N,W", [
    ("bf16", 2, 1, 8),      # one token of one 16-byte piece: only lane 0 holds data
    ("f32", 2, 5, 4),
    ("bf16", 3, 37, 520),   # 65 pieces: the second group of 64 holds one
    ("bf16", 1, 300, 2048), # four pieces per lane
])
def test_gate_widths_and_lengths(marca, dtype, B, N, W):
    x, y, rho = gate_features(B, N, W, seed=B * 1000 + N + W, device=DEV, dtype=dtype)
    cos, reuse, cidx, clen = marca.mar_cos_gate(x, y, 0.95)
    torch.cuda.synchronize()
    c_gpu = cos.double().cpu().numpy()
    tau32 = float(np.float32(0.95))
    r2, c2, l2 = oracle.gate_from_cos(c_gpu, tau32)
    assert (reuse.cpu().numpy() == r2).all() and (cidx.cpu().numpy() == c2).all()
    assert (clen.cpu().numpy() == l2).all()
    c_ref, r_ref, _, _ = oracle.cos_gate(x.double().cpu().numpy(), y.double().cpu().numpy(), tau32)
    assert np.abs(c_gpu - c_ref).max() <= GATE_COS_TOL
    away = np.abs(c_ref - tau32) > 1e-4
    assert (reuse.cpu().numpy()[away] == r_ref[away]).all()


def test_gate_near_threshold(marca):
    x, y, rho = gate_features(2, 300, 1024, seed=22, device=DEV, near_tau=0.95, near_width=1e-3)
    cos, reuse, cidx, clen = marca.mar_cos_gate(x, y, 0.95)
    torch.cuda.synchronize()
    c_gpu = cos.double().cpu().numpy()
    tau32 = float(np.float32(0.95))
    r2, c2, l2 = oracle.gate_from_cos(c_gpu, tau32)
    assert (reuse.cpu().numpy() == r2).all() and (cidx.cpu().numpy() == c2).all()
    c_ref, r_ref, _, _ = oracle.cos_gate(x.double().cpu().numpy(), y.double().cpu().numpy(), tau32)
    assert np.abs(c_gpu - c_ref).max() <= 1e-5  # cosines of the same bf16 values, fp32 sums
    away = np.abs(c_ref - tau32) > 1e-4
    assert away.sum() > 0 and (~away).sum() > 0
    assert (reuse.cpu().numpy()[away] == r_ref[away]).all()


def test_gate_zero_and_parallel_vectors(marca):
    W = 64
    x = torch.zeros((1, 4, W), dtype=torch.float32, device=DEV)
    y = torch.zeros_like(x)
    x[0, 1] = 1.0
    y[0, 1] = 2.0           # parallel -> 1, reuse
    x[0, 2, 0] = 1.0
    y[0, 2, 1] = 1.0        # orthogonal -> 0
    x[0, 3] = 1.0
    y[0, 3] = -1.0          # opposite -> -1
    cos, reuse, cidx, clen = marca.mar_cos_gate(x, y, 0.95)
    torch.cuda.synchronize()
    np.testing.assert_allclose(cos.cpu().numpy()[0], [0, 1, 0, -1], atol=1e-6)
    assert reuse.cpu().numpy()[0].tolist() == [0, 1, 0, 0]
    assert cidx.cpu().numpy()[0].tolist() == [0, 2, 3, -1] and int(clen[0]) == 3
    _, _, _, _, ridx, rlen = gate_with_reuse(marca, x, y)
    torch.cuda.synchronize()
    assert ridx.cpu().numpy()[0].tolist() == [1, -1, -1, -1] and int(rlen[0]) == 1


def test_gate_full_size_highres(marca):
    """512x512-equivalent: 64 sequences x 1088 tokens x W 1024, bf16; sampled oracle rows."""
    B, N, W = 64, 1088, 1024
    x, y, rho = device_gate_features(B, N, W, seed=1005, device=DEV)
    cos, reuse, cidx, clen, ridx, rlen = gate_with_reuse(marca, x, y)
    torch.cuda.synchronize()
    c_gpu = cos.double().cpu().numpy()
    tau32 = float(np.float32(0.95))
    r2, c2, l2 = oracle.gate_from_cos(c_gpu, tau32)
    assert (reuse.cpu().numpy() == r2).all() and (cidx.cpu().numpy() == c2).all()
    assert (clen.cpu().numpy() == l2).all()
    ri, rl = reuse_lists(r2)
    assert (ridx.cpu().numpy() == ri).all() and (rlen.cpu().numpy() == rl).all()
    rows = [0, 17, 63]
    c_ref, r_ref, _, _ = oracle.cos_gate(x[rows].double().cpu().numpy(),
                                         y[rows].double().cpu().numpy(), tau32)
    assert np.abs(c_gpu[rows] - c_ref).max() <= GATE_COS_TOL
    frac = reuse.float().mean().item()
    assert 0.80 < frac < 0.88  # the seeded 84% reuse share


# ---------------------------------------------------------------- CFG ------

@pytest.mark.parametrize("shape", [(64, 256, 16), (3, 7, 5)])
def test_cfg_store_reuse_bit_exact(marca, shape):
    c0, u0, c1, _ = cfg_outputs(*shape, seed=31)
    tc0, tu0, tc1 = (torch.from_numpy(a).to(DEV) for a in (c0, u0, c1))
    guided = torch.empty_like(tc0)
    res, _ = marca.mar_cfg_residual(tc0, tu0, guided_out=guided, cfg_scale=4.0)
    torch.cuda.synchronize()
    rr, rg = oracle.cfg_residual(c0, u0, mode=0, w=4.0)
    assert (res.cpu().numpy() == rr).all()
    g = guided.cpu().numpy().astype(np.float64)
    u64, c64 = u0.astype(np.float64), c0.astype(np.float64)
    exact = u64 + 4.0 * (c64 - u64)
    bound = 2.0 ** -22 * (np.abs(u64) + 2.0 * np.abs(4.0 * (c64 - u64)))  # three roundings
    assert (np.abs(g - exact) <= bound).all()
    guided2 = torch.empty_like(tc0)
    uo, _ = marca.mar_cfg_residual(tc1, residual=res, mode=marca.MAR_CFG_REUSE,
                                   guided_out=guided2, cfg_scale=4.0)
    torch.cuda.synchronize()
    ru, _ = oracle.cfg_residual(c1, residual=rr, mode=1, w=4.0)
    assert (uo.cpu().numpy() == ru).all()


def test_cfg_golden_values(marca, golden_dir):
    import json
    import os
    with open(os.path.join(golden_dir, "cfg_cases.json")) as f:
        g = json.load(f)
    st, ru = g["store"], g["reuse"]
    c = torch.tensor(st["cond"], device=DEV)
    u = torch.tensor(st["uncond"], device=DEV)
    gd = torch.empty_like(c)
    res, _ = marca.mar_cfg_residual(c, u, guided_out=gd, cfg_scale=g["w"])
    c2 = torch.tensor(ru["cond"], device=DEV)
    gd2 = torch.empty_like(c2)
    uo, _ = marca.mar_cfg_residual(c2, residual=torch.tensor(ru["residual"], device=DEV),
                                   mode=marca.MAR_CFG_REUSE, guided_out=gd2, cfg_scale=g["w"])
    torch.cuda.synchronize()
    assert res.tolist() == st["residual"] and gd.tolist() == st["guided"]
    assert uo.tolist() == ru["uncond"] and gd2.tolist() == ru["guided"]
