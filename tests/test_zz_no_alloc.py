"""The allocation-free top-K entry point (mar_refresh_topk_noalloc) against
mar_refresh_topk with a caller workspace, on two calls in a row through the C
ABI, the second smaller than the first (the library's per-device array keeps
the first call's partials; the second must not see them).

Both entry points run the same kernels on the same inputs, so scores and
every index output must be bit-identical; the selection is also checked
against the oracle on the GPU's own scores.
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


def _case(B, H, G, N, n_gp, seed, dtype=torch.bfloat16):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn(B, H, G, 64, device=DEV, generator=gen).to(dtype)
    k = torch.randn(B, H, N, 64, device=DEV, generator=gen).to(dtype)
    perm = torch.stack([torch.randperm(N, device=DEV, generator=gen) for _ in range(B)])
    gp = perm[:, :n_gp].to(torch.int32).contiguous()
    return q, k, gp


def _outs(B, N, n_act):
    return (torch.full((B, N), float("nan"), device=DEV),
            torch.full((B, n_act), -7, dtype=torch.int32, device=DEV),
            torch.full((B, N), -7, dtype=torch.int32, device=DEV),
            torch.full((B,), -7, dtype=torch.int32, device=DEV))


def test_noalloc_matches_workspace_form(marca):
    import oracle
    # (B, H, G, N, |G|+|P|, K): first the MAR-L step's shape (register-resident
    # scores kernel, 2.6 MB of partials), then a smaller call through the
    # LDS scores kernel (20 generating queries) that reuses the array.
    for (B, H, G, N, n_gp, K), seed in (((128, 16, 16, 320, 32, 16), 1),
                                        ((3, 2, 20, 100, 30, 9), 2)):
        print(f"noalloc top-K: B={B} H={H} G={G} N={N} n_gp={n_gp} K={K}", flush=True)
        q, k, gp = _case(B, H, G, N, n_gp, seed)
        ref = marca.mar_refresh_topk(q, k, gp, n_gp, K, *_outs(B, N, n_gp + K))
        got = marca.mar_refresh_topk_noalloc(q, k, gp, n_gp, K, *_outs(B, N, n_gp + K))
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), "scores differ from the workspace form"
        for a, b in zip(got[1:], ref[1:]):
            assert torch.equal(a, b), "indices differ from the workspace form"
        s = got[0].double().cpu().numpy()
        assert np.allclose(s.sum(1), 1.0, atol=1e-4)
        ra, rc, rl = oracle.refresh_select(s, gp.cpu().numpy(), K)
        assert (got[1].cpu().numpy() == ra).all() and (got[2].cpu().numpy() == rc).all()
        assert (got[3].cpu().numpy() == rl).all()


def test_noalloc_rejects_oversized(marca):
    B, H, G, N = 1024, 16, 16, 320  # 20 MiB of partials > the 8 MiB array
    assert B * H * N * 4 > marca.MAR_REFRESH_TOPK_SCRATCH_BYTES
    q = torch.empty((B, H, G, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((B, H, N, 64), dtype=torch.bfloat16, device=DEV)
    gp = torch.zeros((B, 4), dtype=torch.int32, device=DEV)
    with pytest.raises(marca.MarError) as e:
        marca.mar_refresh_topk_noalloc(q, k, gp, 4, 4)
    assert e.value.status == -5  # MAR_E_WORKSPACE
