"""prepare(): a binding call marshalled once and replayed must make the same
library calls as the direct call -- same outputs bit for bit -- and raise
MarError on a failing status as the direct call does (the library's own
argument checks run when the call is made)."""
import pytest
import torch

from mar_workloads import CONFIGS, attention_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def marca():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import cache_aware_attention_amd as m
    return m


def test_prepared_attention_and_update_replay(marca):
    cfg = CONFIGS["mar_l"].__class__(**{**CONFIGS["mar_l"].__dict__, "B": 3, "H": 2})
    x = attention_inputs(cfg, DEV)
    direct = marca.mar_cache_attn_fwd(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                      x["cached"])
    out = torch.full_like(direct, float("nan"))
    call = marca.prepare(marca.mar_cache_attn_fwd, x["q_a"], x["k_a"], x["v_a"], x["k_cache"],
                         x["v_cache"], x["cached"], out=out)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()  # preparing runs nothing
    for _ in range(2):
        out.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, direct)
    # the fused update through a prepared call writes the same cache rows
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    kc2, vc2 = x["k_cache"].clone(), x["v_cache"].clone()
    marca.mar_cache_attn_fwd_update(x["q_a"], x["k_a"], x["v_a"], kc, vc, x["cached"], x["active"])
    o2 = torch.empty_like(direct)
    marca.prepare(marca.mar_cache_attn_fwd_update, x["q_a"], x["k_a"], x["v_a"], kc2, vc2,
                  x["cached"], x["active"], out=o2)()
    torch.cuda.synchronize()
    assert torch.equal(o2, direct) and torch.equal(kc2, kc) and torch.equal(vc2, vc)


def test_prepared_reports_status(marca):
    q = torch.empty((1, 1, 16, 32), dtype=torch.bfloat16, device=DEV)  # head dim 32: unsupported
    with pytest.raises(marca.MarError):
        marca.prepare(marca.mar_cache_attn_fwd, q, q, q, q, q, None, Nc=0)()
