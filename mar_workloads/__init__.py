"""Seeded synthetic inputs shaped like KV-cached MAR decoding.

This module is shared by the GPU tests, the benchmark and the oracle tests.  It
holds no arithmetic of the method itself: only random draws, shapes, the
generation-order permutation and the per-step token counts of the MAR masking
schedule (the latter shapes the workload; the method's own step rules live in
the library and, independently, in the oracle).

Shapes follow the MAR-B/L/H models the method pages evaluate (ImageNet 256x256,
16x16 = 256 image tokens, 64 decoding steps, classifier-free guidance doubling
the batch) plus a tiny CPU-checkable case and a 512x512-equivalent stress case.
No dataset or trained weight is used: values are i.i.d. normal, and the stale
cache is the fresh K/V plus Gaussian noise scaled so that the expected cosine
similarity between a cached and a fresh row is about 0.95, the stability level
the MARche pages report for key/value projections between adjacent steps.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# expected cosine 0.95 between x and x + sigma * n for x, n ~ N(0, I):
# cos ~= 1 / sqrt(1 + sigma^2)  =>  sigma = sqrt(1/0.95^2 - 1)
STALE_SIGMA = math.sqrt(1.0 / 0.95 ** 2 - 1.0)


@dataclass(frozen=True)
class Config:
    name: str
    B: int          # sequences (images x 2 for cond/uncond)
    H: int
    D: int
    N: int          # tokens per sequence (prefix + image)
    n_prefix: int
    A: int          # active tokens per cache-aware step
    n_gen: int
    n_prev: int
    K: int          # refreshing tokens
    layers: int
    dtype: str      # "f32" | "bf16"
    stale: bool     # cached K/V differ from fresh K/V
    steps: int = 64
    budget: int = 0
    W: int = 0      # hidden width (gate features)
    tau: float = 0.95
    cfg_channels: int = 16
    seed: int = 0
    extra: Dict[str, float] = field(default_factory=dict)

    @property
    def B_img(self) -> int:
        return self.B // 2 if self.B > 1 else 1

    @property
    def n_img(self) -> int:
        return self.N - self.n_prefix

    @property
    def Nc(self) -> int:
        return self.N - self.A


CONFIGS: Dict[str, Config] = {
    # 1 sequence, 2 heads, D 64, N 64 (8x8), 8 random active tokens, fp32,
    # cache == fresh (the exact-equivalence case), one cache-aware layer.
    "tiny": Config("tiny", B=1, H=2, D=64, N=64, n_prefix=0, A=8, n_gen=0, n_prev=0, K=0,
                   layers=1, dtype="f32", stale=False, seed=1001),
    # 32 images x 2 CFG, 12 heads x 64, N = 64 prefix + 256 image, active 24 (8+8+8).
    "mar_b": Config("mar_b", B=64, H=12, D=64, N=320, n_prefix=64, A=24, n_gen=8, n_prev=8, K=8,
                    layers=24, dtype="bf16", stale=True, budget=24, W=768, seed=1002),
    # 64 images x 2 CFG, 16 heads x 64, N 320, active 48 = 16 + 16 + top-16.
    "mar_l": Config("mar_l", B=128, H=16, D=64, N=320, n_prefix=64, A=48, n_gen=16, n_prev=16,
                    K=16, layers=32, dtype="bf16", stale=True, budget=48, W=1024, seed=1003),
    # 128 images x 2 CFG, 20 heads x 64, N 320, active budget 64.
    "mar_h": Config("mar_h", B=256, H=20, D=64, N=320, n_prefix=64, A=64, n_gen=16, n_prev=16,
                    K=32, layers=40, dtype="bf16", stale=True, budget=64, W=1280, seed=1004),
    # 512x512-equivalent: 32 images x 2 CFG, 16 heads x 64, N = 64 + 1024, budget 128,
    # cosine gate on W = 1024 features at threshold 0.95.
    "highres": Config("highres", B=64, H=16, D=64, N=1088, n_prefix=64, A=128, n_gen=26,
                      n_prev=26, K=76, layers=32, dtype="bf16", stale=True, budget=128, W=1024,
                      seed=1005),
}


def rng(seed: int, *tags: int) -> np.random.Generator:
    """Independent numpy generator for (seed, tag...)."""
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(t) for t in tags]))


# ---------------------------------------------------------------------------
# MAR generation order and masking schedule (workload shape)
# ---------------------------------------------------------------------------

def cosine_counts(n_img: int, steps: int) -> np.ndarray:
    """Tokens generated per step under MAR's cosine masking schedule.

    After step t (0-based) about floor(n_img * cos(pi/2 * (t+1)/steps)) tokens
    stay masked; every step generates at least one token and the last step
    generates whatever is left.  Sums to n_img.
    """
    counts = []
    remaining = n_img
    for t in range(steps):
        if t == steps - 1:
            n = remaining
        else:
            target = int(math.floor(n_img * math.cos(math.pi / 2.0 * (t + 1) / steps)))
            target = max(1, min(remaining - 1, target))
            n = remaining - target
        counts.append(n)
        remaining -= n
    return np.asarray(counts, dtype=np.int32)


def generation_order(cfg: Config, seed: Optional[int] = None) -> np.ndarray:
    """[B, n_img] token positions (prefix offset applied) in generation order.

    One seeded random permutation per image; the cond and uncond sequences of
    image i (sequences i and i + B_img) share it.
    """
    seed = cfg.seed if seed is None else seed
    orders = np.empty((cfg.B_img, cfg.n_img), np.int32)
    for i in range(cfg.B_img):
        orders[i] = rng(seed, 7, i).permutation(cfg.n_img).astype(np.int32) + cfg.n_prefix
    reps = cfg.B // cfg.B_img
    return np.ascontiguousarray(np.tile(orders, (reps, 1)))


def random_partition(cfg: Config, seed: Optional[int] = None, ascending: bool = True):
    """A seeded active/cached split per sequence for attention-only workloads.

    Returns (active [B, A], cached [B, Nc]) int32.  Active positions are drawn
    from the image range; the cached list holds all other positions, ascending
    or in a seeded random order.  The cond/uncond pair of an image share it.
    """
    seed = cfg.seed if seed is None else seed
    act = np.empty((cfg.B_img, cfg.A), np.int32)
    cac = np.empty((cfg.B_img, cfg.Nc), np.int32)
    for i in range(cfg.B_img):
        g = rng(seed, 11, i)
        pool = np.arange(cfg.n_prefix, cfg.N, dtype=np.int32) if cfg.n_img >= cfg.A \
            else np.arange(cfg.N, dtype=np.int32)
        a = g.choice(pool, size=cfg.A, replace=False).astype(np.int32)
        taken = np.zeros(cfg.N, bool)
        taken[a] = True
        rest = np.nonzero(~taken)[0].astype(np.int32)
        if not ascending:
            rest = g.permutation(rest).astype(np.int32)
        act[i] = a
        cac[i] = rest
    reps = cfg.B // cfg.B_img
    return (np.ascontiguousarray(np.tile(act, (reps, 1))),
            np.ascontiguousarray(np.tile(cac, (reps, 1))))


# ---------------------------------------------------------------------------
# Host (numpy) draws for CPU-sized cases
# ---------------------------------------------------------------------------

def normal(shape, seed: int, *tags: int) -> np.ndarray:
    return rng(seed, *tags).standard_normal(shape)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even), returned as float64.

    Input preparation only: turns a normal draw into values a bf16 tensor holds.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Device (torch) draws for full-size cases
# ---------------------------------------------------------------------------

def torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def device_normal(shape, seed: int, device, dtype, std: float = 1.0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def attention_inputs(cfg: Config, device, seed: Optional[int] = None, ascending: bool = True,
                     A: Optional[int] = None):
    """Seeded inputs of one cache-aware attention layer-call.

    Returns a dict with q_a, k_a, v_a [B,H,A,D], k_cache, v_cache [B,H,N,D],
    active [B,A] and cached [B,Nc] (int32, on `device`).  K_A/V_A are the fresh
    rows at the active positions; the cache holds fresh rows (tiny case) or
    fresh rows plus noise of std STALE_SIGMA.
    """
    import torch
    seed = cfg.seed if seed is None else seed
    if A is not None and A != cfg.A:
        cfg = Config(**{**cfg.__dict__, "A": int(A)})
    dt = torch_dtype(cfg.dtype)
    B, H, N, D = cfg.B, cfg.H, cfg.N, cfg.D
    fresh_k = device_normal((B, H, N, D), seed * 16 + 1, device, torch.float32)
    fresh_v = device_normal((B, H, N, D), seed * 16 + 2, device, torch.float32)
    q_a = device_normal((B, H, cfg.A, D), seed * 16 + 3, device, dt)
    active, cached = random_partition(cfg, seed, ascending)
    act_t = torch.from_numpy(active).to(device=device, dtype=torch.long)
    gather = act_t[:, None, :, None].expand(B, H, cfg.A, D)
    k_a = torch.gather(fresh_k, 2, gather).to(dt)
    v_a = torch.gather(fresh_v, 2, gather).to(dt)
    if cfg.stale:
        k_cache = (fresh_k + device_normal((B, H, N, D), seed * 16 + 4, device, torch.float32,
                                           STALE_SIGMA)).to(dt)
        v_cache = (fresh_v + device_normal((B, H, N, D), seed * 16 + 5, device, torch.float32,
                                           STALE_SIGMA)).to(dt)
    else:
        k_cache = fresh_k.to(dt)
        v_cache = fresh_v.to(dt)
    del fresh_k, fresh_v
    return {
        "q_a": q_a.contiguous(), "k_a": k_a.contiguous(), "v_a": v_a.contiguous(),
        "k_cache": k_cache.contiguous(), "v_cache": v_cache.contiguous(),
        "active": torch.from_numpy(active).to(device),
        "cached": torch.from_numpy(cached).to(device),
        "cfg": cfg,
    }


def gate_features(B: int, N: int, W: int, seed: int, device=None, dtype: str = "bf16",
                  reuse_frac: float = 0.84, rho_hi: float = 0.99, rho_lo: float = 0.80,
                  near_tau: Optional[float] = None, near_width: float = 1e-3):
    """(x_cur, x_cached, rho) with a target cosine per token.

    x_cached ~ N(0, I_W); x_cur = |x| (rho * xhat + sqrt(1 - rho^2) * u) with u a
    random unit vector orthogonal to xhat.  rho = rho_hi for a seeded
    `reuse_frac` of tokens (the share of skipped tokens LazyMAR reports) and
    rho_lo for the rest; with near_tau set, rho is drawn within +-near_width of
    it instead (boundary cases).  Built in float64 on the host in blocks.
    """
    g = rng(seed, 23)
    y = g.standard_normal((B, N, W))
    if near_tau is not None:
        rho = near_tau + g.uniform(-near_width, near_width, size=(B, N))
    else:
        hi = g.random((B, N)) < reuse_frac
        rho = np.where(hi, rho_hi, rho_lo)
    u = g.standard_normal((B, N, W))
    yn = np.linalg.norm(y, axis=-1, keepdims=True)
    yhat = y / yn
    u = u - np.sum(u * yhat, axis=-1, keepdims=True) * yhat
    u = u / np.linalg.norm(u, axis=-1, keepdims=True)
    x = yn * (rho[..., None] * yhat + np.sqrt(1.0 - rho[..., None] ** 2) * u)
    if device is None:
        if dtype == "bf16":
            return to_bf16_values(x), to_bf16_values(y), rho
        return x.astype(np.float32).astype(np.float64), y.astype(np.float32).astype(np.float64), rho
    import torch
    dt = torch_dtype(dtype)
    return (torch.from_numpy(x.astype(np.float32)).to(device=device, dtype=dt),
            torch.from_numpy(y.astype(np.float32)).to(device=device, dtype=dt), rho)


def device_gate_features(B: int, N: int, W: int, seed: int, device, dtype: str = "bf16",
                         reuse_frac: float = 0.84, rho_hi: float = 0.99, rho_lo: float = 0.80):
    """Same recipe as gate_features, drawn on the device (for full-size runs)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 31 + 23)
    y = torch.randn((B, N, W), generator=gen, device=device, dtype=torch.float32)
    u = torch.randn((B, N, W), generator=gen, device=device, dtype=torch.float32)
    hi = torch.rand((B, N), generator=gen, device=device) < reuse_frac
    rho = torch.where(hi, torch.tensor(rho_hi, device=device), torch.tensor(rho_lo, device=device))
    yn = torch.linalg.vector_norm(y, dim=-1, keepdim=True)
    yhat = y / yn
    u = u - (u * yhat).sum(-1, keepdim=True) * yhat
    u = u / torch.linalg.vector_norm(u, dim=-1, keepdim=True)
    x = yn * (rho[..., None] * yhat + torch.sqrt(1.0 - rho[..., None] ** 2) * u)
    dt = torch_dtype(dtype)
    return x.to(dt).contiguous(), y.to(dt).contiguous(), rho


def cfg_outputs(B_img: int, T: int, C: int, seed: int):
    """(cond_prev, uncond_prev, cond_now, uncond_now) float32 [B_img, T, C].

    cond drifts by N(0,1) per step while the residual cond - uncond drifts by
    N(0, 1/35.5) (LazyMAR reports the residual changing about 35.5x less than
    either branch between adjacent steps; used here only to shape the data).
    """
    g = rng(seed, 31)
    shape = (B_img, T, C)
    cond0 = g.standard_normal(shape)
    res0 = g.standard_normal(shape)
    cond1 = cond0 + g.standard_normal(shape)
    res1 = res0 + g.standard_normal(shape) / math.sqrt(35.5)
    f = np.float32
    return ((cond0).astype(f), (cond0 - res0).astype(f), (cond1).astype(f),
            (cond1 - res1).astype(f))
