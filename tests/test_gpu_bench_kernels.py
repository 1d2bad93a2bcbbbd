"""The measurement kernels of libmarca_bench on the GPU: the concatenation
that standard attention needs is a bit-exact row copy (a skipped entry leaves
its row as it was), and the attention's memory-operations-only kernel writes
nothing outside its output rows (and nothing at all when told to only read)."""
import numpy as np
import pytest
import torch

from mar_workloads import CONFIGS, attention_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def bench():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import cache_aware_attention_amd  # noqa: F401  (loads libmarca first)
    from cache_aware_attention_amd import _bench_lib
    return _bench_lib


def small(A, B=3, H=2):
    cfg = CONFIGS["mar_l"].__class__(**{**CONFIGS["mar_l"].__dict__, "B": B, "H": H})
    return attention_inputs(cfg, DEV, A=A), cfg


@pytest.mark.parametrize("A", [48, 128])
def test_concat_bit_exact(bench, A):
    x, cfg = small(A)
    Nc = cfg.N - A
    cached = x["cached"].clone()
    cached[1, 5] = -1       # a skipped entry: its row keeps the sentinel
    cached[2, 0] = cfg.N    # out of range: skipped as well
    kcat = torch.full((cfg.B, cfg.H, cfg.N, cfg.D), 7.0, dtype=torch.bfloat16, device=DEV)
    vcat = kcat.clone()
    bench.mar_bench_kv_concat(x["k_a"], x["v_a"], x["k_cache"], x["v_cache"], cached, Nc,
                              kcat, vcat)
    torch.cuda.synchronize()
    i16 = lambda t: t.view(torch.int16).cpu().numpy()
    ka, va, kc, vc = (i16(x[k]) for k in ("k_a", "v_a", "k_cache", "v_cache"))
    cl = cached.cpu().numpy()
    exp_k = np.full(i16(kcat).shape, i16(torch.tensor(7.0, dtype=torch.bfloat16)), np.int16)
    exp_v = exp_k.copy()
    exp_k[:, :, :A], exp_v[:, :, :A] = ka, va
    for b in range(cfg.B):
        for j in range(Nc):
            n = cl[b, j]
            if 0 <= n < cfg.N:
                exp_k[b, :, A + j], exp_v[b, :, A + j] = kc[b, :, n], vc[b, :, n]
    assert (i16(kcat) == exp_k).all() and (i16(vcat) == exp_v).all()


def test_pattern_kernel_writes_only_its_rows(bench):
    x, cfg = small(48)
    B, H, A, D = x["q_a"].shape
    sentinel = -12345
    buf = torch.full((B * H * A * D + 4096,), sentinel, dtype=torch.int16, device=DEV)
    out = buf[:B * H * A * D].view(torch.bfloat16).view(B, H, A, D)
    bench.mar_bench_attn_pattern(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                 x["cached"], cfg.Nc, out, write_out=False)
    torch.cuda.synchronize()
    assert (buf == sentinel).all()
    bench.mar_bench_attn_pattern(x["q_a"], x["k_a"], x["v_a"], x["k_cache"], x["v_cache"],
                                 x["cached"], cfg.Nc, out, write_out=True)
    torch.cuda.synchronize()
    assert (buf[B * H * A * D:] == sentinel).all()
    # every 16-byte piece of the output rows was written
    pieces = buf[:B * H * A * D].view(-1, 8)
    assert not (pieces == sentinel).all(dim=1).any()


def test_dense_floor_modes(bench):
    """The full-attention kernel's measurement modes: the arithmetic-only mode
    stores nothing (no memory traffic), the memory-only mode writes every
    output row; both leave everything past the output untouched."""
    from mar_workloads import device_normal
    B, H, N, D = 2, 3, 400, 64
    q, k, v = (device_normal((B, H, N, D), 90 + i, DEV, torch.bfloat16) for i in range(3))
    sentinel = -12345
    buf = torch.full((B * H * N * D + 4096,), sentinel, dtype=torch.int16, device=DEV)
    out = buf[:B * H * N * D].view(torch.bfloat16).view(B, H, N, D)
    bench.mar_bench_dense_floor(q, k, v, out, bench.MAR_BENCH_FLOOR_ARITH)
    torch.cuda.synchronize()
    assert (buf == sentinel).all()
    bench.mar_bench_dense_floor(q, k, v, out, bench.MAR_BENCH_FLOOR_MEMORY)
    torch.cuda.synchronize()
    assert (buf[B * H * N * D:] == sentinel).all()
    pieces = buf[:B * H * N * D].view(-1, 8)
    assert not (pieces == sentinel).all(dim=1).any()


def test_refresh_floor_modes(bench):
    """The refresh-step layer's measurement modes: the arithmetic-only mode
    writes neither the output nor the caches; the memory-only mode rewrites
    every cache row with the fresh K/V, as the layer does."""
    from mar_workloads import device_normal
    B, H, N, D = 2, 3, 400, 64
    q, k, v = (device_normal((B, H, N, D), 95 + i, DEV, torch.bfloat16) for i in range(3))
    kc = torch.full((B, H, N, D), 5.0, dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, 5.0)
    out = torch.full_like(kc, 7.0)
    bench.mar_bench_dense_floor(q, k, v, out, bench.MAR_BENCH_FLOOR_ARITH, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    assert (kc == 5.0).all() and (vc == 5.0).all() and (out == 7.0).all()
    bench.mar_bench_dense_floor(q, k, v, out, bench.MAR_BENCH_FLOOR_MEMORY, k_cache=kc, v_cache=vc)
    torch.cuda.synchronize()
    assert torch.equal(kc, k) and torch.equal(vc, v)


def test_cached_floor_modes(bench):
    """The cached workgroup kernel's measurement modes, uniform counts: the
    arithmetic-only mode writes nothing; the memory-only mode writes every
    output row and nothing past the output."""
    from mar_workloads import device_normal
    B, H, N, A, D = 2, 3, 600, 96, 64
    Nc = N - A
    q, k, v = (device_normal((B, H, A, D), 70 + i, DEV, torch.bfloat16) for i in range(3))
    kc, vc = (device_normal((B, H, N, D), 73 + i, DEV, torch.bfloat16) for i in range(2))
    g = torch.Generator().manual_seed(7)
    cidx = torch.stack([torch.randperm(N, generator=g)[:Nc] for _ in range(B)]).to(torch.int32)
    cidx = cidx.to(DEV)
    sentinel = -12345
    buf = torch.full((B * H * A * D + 4096,), sentinel, dtype=torch.int16, device=DEV)
    out = buf[:B * H * A * D].view(torch.bfloat16).view(B, H, A, D)
    bench.mar_bench_cached_floor(q, k, v, kc, vc, cidx, out, bench.MAR_BENCH_FLOOR_ARITH)
    torch.cuda.synchronize()
    assert (buf == sentinel).all()
    bench.mar_bench_cached_floor(q, k, v, kc, vc, cidx, out, bench.MAR_BENCH_FLOOR_MEMORY)
    torch.cuda.synchronize()
    assert (buf[B * H * A * D:] == sentinel).all()
    pieces = buf[:B * H * A * D].view(-1, 8)
    assert not (pieces == sentinel).all(dim=1).any()


def test_cached_floor_modes_ragged_update(bench):
    """The same modes for the per-sequence layer with the cache update: the
    arithmetic-only mode writes neither the output nor the caches; the
    memory-only mode writes each sequence's first a_len rows of k_a/v_a into
    the caches at active_idx (nothing else) and only its first a_len output
    rows."""
    from mar_workloads import device_normal
    B, H, N, A, D = 3, 2, 500, 150, 64
    q, k, v = (device_normal((B, H, A, D), 80 + i, DEV, torch.bfloat16) for i in range(3))
    a_len = torch.tensor([150, 97, 140], dtype=torch.int32)
    g = torch.Generator().manual_seed(11)
    act = torch.full((B, A), -1, dtype=torch.int32)
    cid = torch.full((B, N), -1, dtype=torch.int32)
    for b in range(B):
        perm = torch.randperm(N, generator=g).to(torch.int32)
        n = int(a_len[b])
        act[b, :n] = perm[:n]
        cid[b, :N - n] = torch.sort(perm[n:]).values
    c_len = (N - a_len).to(torch.int32)
    act, cid, a_len, c_len = (t.to(DEV) for t in (act, cid, a_len, c_len))
    kc = torch.full((B, H, N, D), 5.0, dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, 5.0)
    out = torch.full_like(q, 7.0)
    bench.mar_bench_cached_floor(q, k, v, kc, vc, cid, out, bench.MAR_BENCH_FLOOR_ARITH,
                                 active_idx=act, a_len=a_len, c_len=c_len)
    torch.cuda.synchronize()
    assert (kc == 5.0).all() and (vc == 5.0).all() and (out == 7.0).all()
    bench.mar_bench_cached_floor(q, k, v, kc, vc, cid, out, bench.MAR_BENCH_FLOOR_MEMORY,
                                 active_idx=act, a_len=a_len, c_len=c_len)
    torch.cuda.synchronize()
    ek = torch.full_like(kc, 5.0)
    ev = torch.full_like(vc, 5.0)
    for b in range(B):
        n = int(a_len[b])
        pos = act[b, :n].long()
        ek[b][:, pos] = k[b, :, :n]
        ev[b][:, pos] = v[b, :, :n]
        assert (out[b, :, n:] == 7.0).all()
        assert not (out[b, :, :n] == 7.0).all(dim=-1).any()
    assert torch.equal(kc, ek) and torch.equal(vc, ev)
