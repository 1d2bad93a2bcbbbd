"""Layer 2's full attention with the refresh partials (mar_cache_attn_fwd_scores)
and the selection from them (mar_refresh_select), against the oracle.

- The attention output is the full attention's, bit for bit the output of
  mar_cache_attn_fwd on the same inputs (the same main loop).
- The per-head partials are the generating queries' softmax probabilities
  summed over those queries: within normwise relative 1e-5 of the oracle's
  fp64 refresh scores of each head (scaled by G), and the selection's scores
  (their mean over heads and queries) likewise.
- The selection is bit-exact against the oracle's selection on the GPU's own
  scores (where floating point decides an integer, both sides decide on the
  same floats).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def marca():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import cache_aware_attention_amd as m
    return m


def f64(t):
    return t.detach().double().cpu().numpy()


def make(B, H, N, G, n_gp, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    q, k, v = (torch.randn(B, H, N, 64, device=DEV, generator=g).to(torch.bfloat16)
               for _ in range(3))
    perm = torch.stack([torch.randperm(N, device=DEV, generator=g) for _ in range(B)])
    gp = perm[:, :n_gp].to(torch.int32).contiguous()       # previous tokens, then generating
    gen = gp[:, n_gp - G:].contiguous()                   # the generating tokens
    return q, k, v, gp, gen


def check(marca, q, k, v, gp, gen, G, K, rows=None):
    import oracle
    B, H, N, D = q.shape
    n_gp = gp.shape[1]
    out, part = marca.mar_cache_attn_fwd_scores(q, k, v, gen, G)
    ref_out = marca.mar_cache_attn_fwd(q, k, v, k, v, None, Nc=0)
    scores, act, cac, clen = marca.mar_refresh_select(part, gp, n_gp, K, G)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "the attention output differs from the full attention's"
    rows = list(range(B)) if rows is None else rows
    gcpu = gen.cpu().numpy()
    qn, kn, pn = f64(q), f64(k), f64(part)
    for b in rows:
        valid = [int(p) for p in gcpu[b] if 0 <= p < N]
        qg = qn[b:b + 1, :, valid]                       # [1,H,Gv,D]
        for h in range(H):
            ref_h = oracle.refresh_scores(qg[:, h:h + 1], kn[b:b + 1, h:h + 1], D ** -0.5)[0]
            ref_h *= len(valid)                          # sums over the valid generating queries
            err = np.abs(pn[b, h] - ref_h).max() / np.abs(ref_h).max()
            assert err <= 1e-5, (b, h, err)
        ref_s = oracle.refresh_scores(qg, kn[b:b + 1], D ** -0.5)[0] * len(valid) / G
        s = f64(scores)[b]
        assert np.abs(s - ref_s).max() / np.abs(ref_s).max() <= 1e-5
    ra, rc, rl = oracle.refresh_select(f64(scores), gp.cpu().numpy(), K)
    assert (act.cpu().numpy() == ra).all() and (cac.cpu().numpy() == rc).all()
    assert (clen.cpu().numpy() == rl).all()
    return scores


@pytest.mark.parametrize("B,H,N,G,n_gp,K,seed", [
    (3, 4, 320, 16, 32, 16, 1),   # the MAR-L step's shape per sequence
    (2, 3, 300, 5, 11, 20, 2),    # a partial last chunk, fewer than 16 generating queries
    (2, 2, 96, 1, 1, 7, 3),       # three chunks, one generating query
])
def test_scores_and_selection(marca, B, H, N, G, n_gp, K, seed):
    q, k, v, gp, gen = make(B, H, N, G, n_gp, seed)
    scores = check(marca, q, k, v, gp, gen, G, K)
    assert torch.allclose(scores.sum(1), torch.ones(B, device=DEV), atol=1e-4)


def test_invalid_generating_entry_contributes_nothing(marca):
    q, k, v, gp, gen = make(2, 2, 320, 6, 12, 4)
    gen = gen.clone()
    gen[1, 2] = -1
    gen[0, 5] = 320
    scores = check(marca, q, k, v, gp, gen, 6, 10)
    # each sequence lost one of its six queries: its scores sum to 5/6
    assert torch.allclose(scores.sum(1), torch.full((2,), 5 / 6, device=DEV), atol=1e-4)


def test_strided_generating_list(marca):
    """The generating tokens as a column slice of a wider index list (row
    stride != G), as a decode passes a slice of the generation order."""
    q, k, v, gp, gen = make(2, 2, 320, 8, 24, 6)
    wide = torch.full((2, 40), -1, dtype=torch.int32, device=DEV)
    wide[:, 24:32] = gen
    check(marca, q, k, v, gp, wide[:, 24:32], 8, 12)


def test_full_size_mar_l(marca):
    """128 sequences x 16 heads, N = 320, G = 16: sampled sequences against the
    oracle; every sequence's scores sum to 1 and its partition covers every token."""
    q, k, v, gp, gen = make(128, 16, 320, 16, 32, 5)
    scores = check(marca, q, k, v, gp, gen, 16, 16, rows=[0, 77, 127])
    assert torch.allclose(scores.sum(1), torch.ones(128, device=DEV), atol=1e-4)
