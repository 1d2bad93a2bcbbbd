"""Benchmark: one KV-cached MAR decode step of the cache-aware path at the MAR-L shape.

A "step" is one non-refresh decoding step of a MAR-L-like model (64 images x 2
CFG = 128 sequences, 16 heads x 64, N = 320 tokens, active 48 = 16 generating
+ 16 previous + 16 refreshing, 32 layers) through every row of the hot path:

  * the host step plan (refresh decision, budget-filled K);
  * layer 2: refresh scores + top-K + active/cached partition (mar_refresh_topk);
  * layers 3..32 (30 layers): cache-aware attention fused with the cache update
    of the active rows (mar_cache_attn_fwd_update: one operator reads the fresh
    active rows and the stored cached rows, merges the two softmax sums, and
    writes the fresh rows into that layer's cache);
  * the CFG condition cache reuse on the 16-channel token outputs (mar_cfg_residual);
  * one cosine-gate evaluation on the 1024-wide hidden features (mar_cos_gate).

The same step with the attention (mar_cache_attn_fwd) and the K/V scatter
(mar_kv_scatter_refresh, on a second stream) as separate kernels is timed
beside it (`unfused_step`).

Every layer owns distinct Q/K/V and cache buffers (about 6.5 GB in all), so the
256 MB Infinity Cache cannot serve one layer's data to the next.  Inputs are
seeded synthetic tensors already resident in HBM.

Prints ONE JSON line.  `value` = active-query tokens per second through the
cache-aware layers (128 x 48 x 30 per step / step time).  `roofline` describes
the dominant kernel of the step (the fused cache-aware attention + cache
update); its average launch duration is measured with HIP events on the
launch stream around groups of 30 back-to-back launches.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "cache-aware attn active-query tok/s + HBM GB/s (% peak), MAR-L-like shape"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_mar_l_traffic.json")
DECODE_ROUNDS = 3
# The attention kernels' sources: the counter record is valid for these bytes only.
ATTN_SRC = tuple(os.path.join(ROOT, "cache_aware_attention_amd", "csrc", f)
                 for f in ("cache_attn.hip", "attn_dense.h"))


def attn_bytes(B, H, A, Nc, D, elem=2):
    """Algorithmic bytes of one cache-aware attention call: read Q_A, K_A, V_A,
    write out (4 x A rows), read the Nc cached K and V rows, read the cached
    index list once per sequence."""
    return B * H * (4 * A + 2 * Nc) * D * elem + B * Nc * 4


def fused_bytes(B, H, A, Nc, D, elem=2):
    """Algorithmic bytes of one fused call (attention + cache update of the
    active rows): the attention's bytes plus the A fresh K and V rows written
    into the caches (they were already read for the attention)."""
    return attn_bytes(B, H, A, Nc, D, elem) + 2 * B * H * A * D * elem


def ragged_update_bytes(H, N, D, counts, elem=2):
    """Algorithmic bytes of mar_cache_attn_fwd_ragged_update over all N tokens
    of each sequence, a[b] = counts[b] of them recomputed: their fresh Q, K, V
    read and out written (4 a rows), the reused tokens' cached K and V read
    (2 (N - a) rows), the recomputed rows' K and V written into the caches
    (2 a rows), per head; and each sequence's N-entry int32 reuse list."""
    return sum(H * (4 * a + 2 * N) * D * elem for a in counts) + len(counts) * N * 4


def headline_record(cfg, n_ca, steps, warmup, ms_per_step, achieved_gbs, traffic, cpu):
    """The required part of the one-line JSON record.  `value` is active-query
    tokens per second of the whole step: B x A queries in each of the n_ca
    cache-aware layers, over the step time.  `roofline` is that of the step's
    dominant kernel, the fused cache-aware attention + cache update:
    `achieved_gbs` is its algorithmic bytes per launch over its measured
    launch time, against the HBM peak."""
    tokens_per_step = cfg.B * cfg.A * n_ca
    return {
        "metric": METRIC, "value": tokens_per_step / (ms_per_step * 1e-3), "unit": "tok/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal Q/K/V, cache = fresh + noise at cosine ~0.95)",
        "config": {"workload": "mar_l_decode_step", "sequences": cfg.B, "heads": cfg.H,
                   "head_dim": cfg.D, "tokens": cfg.N, "active": cfg.A, "cached": cfg.Nc,
                   "cache_aware_layers": n_ca, "refresh_k": cfg.K, "gate_width": cfg.W,
                   "cfg_residual": [cfg.B_img, cfg.n_img, cfg.cfg_channels]},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / PEAK_HBM_GBS, "traffic": traffic},
        "cpu_baseline": cpu,
    }


RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # 312.5


def roofline_for(flops, nbytes, seconds):
    """Roofline entry of a kernel that does `flops` over `nbytes` of algorithmic
    HBM traffic in `seconds`: HBM-bound when its intensity is below the bf16
    matrix-core ridge (peak flop/s over peak bytes/s), matrix-core-bound above."""
    intensity = flops / nbytes
    if intensity < RIDGE_FLOP_PER_BYTE:
        achieved = nbytes / seconds / 1e9
        r = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        achieved = flops / seconds / 1e12
        r = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    r.update({"frac": achieved / r["peak"], "flop_per_byte": intensity,
              "ridge_flop_per_byte": RIDGE_FLOP_PER_BYTE, "flops_per_call": flops,
              "bytes_per_call": nbytes})
    return r


def source_hash(paths):
    """sha256 (first 16 hex digits) of one file, or of several files' bytes in order."""
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kind):
    """Counter-measured HBM bytes per launch of the kernel `kind` ("fused" or
    "attention"), if the counters were taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != source_hash(ATTN_SRC):
        return None
    return t.get("kernels", {}).get(kind, {}).get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x, plan_nc, cfg, args, budget_s=12.0):
    """The oracle on a bounded sample of the step: the top-K, the CFG residual and
    the gate once, then whole layer-calls of the attention (all 2048 (b,h) units)
    and of the scatter, layer after layer, until about `budget_s` seconds of CPU
    work are spent; step time = fixed parts + 30 x the mean per-layer time."""
    import numpy as np
    import torch

    import oracle
    nt = oracle.num_threads()
    t64 = lambda t: t.detach().double().cpu().numpy()
    b16 = lambda t: t.detach().view(torch.int16).cpu().numpy()
    spent = 0.0
    qg, kf = t64(x["q_gen"]), t64(x["k_full"])
    gp = x["gp"].cpu().numpy()
    t0 = time.perf_counter()
    s = oracle.refresh_scores(qg, kf, cfg.D ** -0.5)
    oracle.refresh_select(s, gp, cfg.K)
    t_topk = time.perf_counter() - t0
    del qg, kf
    c, r = x["cond"].cpu().numpy(), x["residual"].cpu().numpy()
    t0 = time.perf_counter()
    oracle.cfg_residual(c, residual=r, mode=1)
    t_cfg = time.perf_counter() - t0
    xg, yg = t64(x["gate_x"]), t64(x["gate_y"])
    t0 = time.perf_counter()
    oracle.cos_gate(xg, yg, float(np.float32(0.95)))
    t_gate = time.perf_counter() - t0
    spent = t_topk + t_cfg + t_gate
    cidx = x["cached_idx"].cpu().numpy()
    act = x["active_idx"].cpu().numpy()
    t_attn, t_scatter, n_layers = 0.0, 0.0, 0
    for L in x["layers"]:
        q, ka, va = t64(L["q_a"]), t64(L["k_a"]), t64(L["v_a"])
        kc, vc = t64(L["k_cache"]), t64(L["v_cache"])
        t0 = time.perf_counter()
        oracle.cache_attention(q, ka, va, kc, vc, cidx, cfg.D ** -0.5, Nc=plan_nc)
        t_attn += time.perf_counter() - t0
        del q, ka, va, kc, vc
        kcb, vcb, kab, vab = (b16(L[k]) for k in ("k_cache", "v_cache", "k_a", "v_a"))
        t0 = time.perf_counter()
        oracle.kv_scatter(kcb, vcb, kab, vab, act)
        t_scatter += time.perf_counter() - t0
        n_layers += 1
        if spent + t_attn + t_scatter >= budget_s:
            break
    n_ca = cfg.layers - 2
    per_layer = (t_attn + t_scatter) / n_layers
    t_step = t_topk + t_cfg + t_gate + n_ca * per_layer
    tokens = cfg.B * cfg.A * n_ca
    return {
        "value": tokens / t_step, "unit": "tok/s", "cores": nt, "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{n_layers} MAR-L layer-calls of attention (2048 (b,h) units each) and of "
                   f"the scatter, plus top-K, CFG residual and gate once; step time = fixed + "
                   f"{n_ca} x mean per-layer ({spent + t_attn + t_scatter:.1f} s of CPU work)"),
        "seconds": {"attn_per_layer": t_attn / n_layers, "scatter_per_layer": t_scatter / n_layers,
                    "topk": t_topk, "cfg": t_cfg, "gate": t_gate, "step_extrapolated": t_step},
    }


def build_inputs(cfg, dev):
    import numpy as np
    import torch

    from mar_workloads import (attention_inputs, cfg_outputs, device_gate_features,
                               device_normal, generation_order)
    import cache_aware_attention_amd as marca

    n_ca = cfg.layers - 2
    layers = []
    for l in range(n_ca):
        x = attention_inputs(cfg, dev, seed=cfg.seed * 100 + l)
        x.pop("cfg")
        x["out"] = torch.empty_like(x["q_a"])
        layers.append(x)
        torch.cuda.synchronize()
    order = torch.from_numpy(generation_order(cfg)).to(dev)
    # a mid-decode step with 16 previous and 16 generating tokens: P then G is one slice
    prev_begin = 96
    gp = order[:, prev_begin:prev_begin + cfg.n_prev + cfg.n_gen]
    q_gen = device_normal((cfg.B, cfg.H, cfg.n_gen, cfg.D), 71, dev, torch.bfloat16)
    k_full = device_normal((cfg.B, cfg.H, cfg.N, cfg.D), 72, dev, torch.bfloat16)
    c0, u0, c1, _ = cfg_outputs(cfg.B_img, cfg.n_img, cfg.cfg_channels, seed=cfg.seed)
    gx, gy, _ = device_gate_features(cfg.B, cfg.N, cfg.W, seed=cfg.seed, device=dev)
    x = {
        "layers": layers, "gp": gp, "q_gen": q_gen, "k_full": k_full,
        "scores": torch.empty((cfg.B, cfg.N), dtype=torch.float32, device=dev),
        "active_idx": torch.empty((cfg.B, cfg.A), dtype=torch.int32, device=dev),
        "cached_idx": torch.empty((cfg.B, cfg.N), dtype=torch.int32, device=dev),
        "cached_len": torch.empty((cfg.B,), dtype=torch.int32, device=dev),
        "workspace": torch.empty((marca.mar_refresh_topk_workspace(cfg.B, cfg.H, cfg.N) // 4,),
                                 dtype=torch.float32, device=dev),
        "cond": torch.from_numpy(c1).to(dev),
        "residual": torch.from_numpy(c0 - u0).to(dev),
        "uncond_out": torch.empty(c1.shape, dtype=torch.float32, device=dev),
        "gate_x": gx, "gate_y": gy,
        "cos": torch.empty((cfg.B, cfg.N), dtype=torch.float32, device=dev),
        "reuse": torch.empty((cfg.B, cfg.N), dtype=torch.uint8, device=dev),
        "cidx": torch.empty((cfg.B, cfg.N), dtype=torch.int32, device=dev),
        "clen": torch.empty((cfg.B,), dtype=torch.int32, device=dev),
        "full_out": torch.empty((cfg.B, cfg.H, cfg.N, cfg.D), dtype=torch.bfloat16, device=dev),
    }
    x["partials"] = x["workspace"].view(cfg.B, cfg.H, cfg.N)
    torch.cuda.synchronize()
    return x


SEQ_KEYS = ("gp", "q_gen", "k_full", "scores", "active_idx", "cached_idx", "cached_len",
            "gate_x", "gate_y", "cos", "reuse", "cidx", "clen", "full_out", "partials")


def seq_view(x, nb):
    """The first nb sequences of every per-sequence tensor of the step (views of
    the same memory).  The conditional branch of each image's CFG pair comes
    first in the batch, so nb = B/2 is the conditional branch alone."""
    v = dict(x)
    for k in SEQ_KEYS:
        v[k] = x[k][:nb]
    v["layers"] = [{k: t[:nb] for k, t in L.items()} for L in x["layers"]]
    return v


def time_rotating(fn, items, stream, R=5, warm_s=0.05):
    """Per-call time of fn over the rotating items: a warm-up of at least
    warm_s seconds, then HIP events on `stream` around R passes."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for it in items:
            fn(it)
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(R):
        for it in items:
            fn(it)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (R * len(items))


LOCALITY_SPLITS = (48, 128)  # active tokens of 320; the rest are cached
LOCALITY_LAYERS = 8


def locality_inputs(marca, dev, A, stream):
    """LOCALITY_LAYERS distinct MAR-L layer-calls with A active of 320 tokens,
    each with prepared calls of: the cache-aware attention (cached rows
    gathered through the list), the concatenation [active ; cached] of
    standard attention, and the same attention kernel over the concatenated
    rows (the list then names contiguous rows A .. 319 of the concatenation)."""
    import torch

    from cache_aware_attention_amd import _bench_lib
    from mar_workloads import CONFIGS, attention_inputs
    cfg = CONFIGS["mar_l"]
    Nc = cfg.N - A
    layers = []
    for l in range(LOCALITY_LAYERS):
        x = attention_inputs(cfg, dev, seed=cfg.seed * 100 + 70 + l, A=A)
        x["out"] = torch.empty_like(x["q_a"])
        x["kcat"] = torch.empty_like(x["k_cache"])
        x["vcat"] = torch.empty_like(x["v_cache"])
        x["contig"] = (torch.arange(A, cfg.N, dtype=torch.int32, device=dev)
                       .expand(cfg.B, Nc).contiguous())
        x["p_ca"] = marca.prepare(marca.mar_cache_attn_fwd, x["q_a"], x["k_a"], x["v_a"],
                                  x["k_cache"], x["v_cache"], x["cached"], Nc=Nc, out=x["out"],
                                  stream=stream)
        x["p_cat"] = marca.prepare(_bench_lib.mar_bench_kv_concat, x["k_a"], x["v_a"],
                                   x["k_cache"], x["v_cache"], x["cached"], Nc, x["kcat"],
                                   x["vcat"], stream=stream)
        x["p_std"] = marca.prepare(marca.mar_cache_attn_fwd, x["q_a"], x["k_a"], x["v_a"],
                                   x["kcat"], x["vcat"], x["contig"], Nc=Nc, out=x["out"],
                                   stream=stream)
        layers.append(x)
    torch.cuda.synchronize()
    return cfg, layers


def locality(marca, dev, stream):
    """The pages' comparison of standard attention (physically concatenating
    the cached and the fresh K/V, then attending) with cache-aware attention
    (no concatenation), at equal work: one MAR-L layer-call (128 sequences x
    16 heads, 320 tokens) with A = 48 and A = 128 active tokens.  Reports the
    cache-aware call, the concatenation, and the same attention kernel over
    the concatenated (contiguous) rows; standard = concatenation + attention.
    Also the same attention with only the cached rows' order changed, which
    is what memory locality alone is worth to the attention."""
    import torch
    res = []
    for A in LOCALITY_SPLITS:
        cfg, layers = locality_inputs(marca, dev, A, stream)
        Nc = cfg.N - A
        for x in layers:
            x["p_cat"]()  # the concatenations exist before the contiguous attention runs
        t_ca = time_rotating(lambda x: x["p_ca"](), layers, stream)
        t_cat = time_rotating(lambda x: x["p_cat"](), layers, stream)
        t_contig = time_rotating(lambda x: x["p_std"](), layers, stream)
        res.append({"active": A, "cached": Nc, "cache_aware_us": t_ca, "concat_us": t_cat,
                    "attention_on_concat_us": t_contig, "standard_us": t_cat + t_contig,
                    "standard_over_cache_aware": (t_cat + t_contig) / t_ca,
                    "contiguous_over_gathered": t_contig / t_ca,
                    "concat_bytes": 2 * 2 * cfg.B * cfg.H * (A + Nc) * cfg.D * 2 + cfg.B * Nc * 4})
        del layers
        torch.cuda.empty_cache()
    return {"what": "standard attention (concatenate [active ; cached] K/V, then attend) vs "
                    "cache-aware attention, one MAR-L layer-call per split",
            "splits": res}


def other_configs(marca, dev, stream):
    """The cache-aware attention call (and, at the high-res length, the full
    attention and refresh-step calls) at the other configurations' shapes:
    time per call over rotating layers whose working set is well above the
    256 MB last-level cache, HIP events around R passes after a warm-up."""
    import torch

    from mar_workloads import CONFIGS, attention_inputs
    res = {}
    for name, n_layers in (("mar_b", 12), ("mar_h", 4), ("highres", 6), ("mar_l_f32", 4)):
        if name == "mar_l_f32":  # the MAR-L shape with fp32 inputs (the per-unit vector path)
            cfg = CONFIGS["mar_l"].__class__(**{**CONFIGS["mar_l"].__dict__, "dtype": "f32"})
        else:
            cfg = CONFIGS[name]
        layers = []
        for l in range(n_layers):
            x = attention_inputs(cfg, dev, seed=cfg.seed * 100 + 50 + l)
            x["out"] = torch.empty_like(x["q_a"])
            layers.append(x)
        torch.cuda.synchronize()

        def timed(fn, R=5):
            # warm up for at least 50 ms: right after the inputs are built the
            # first passes run measurably slower
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.05:
                for L in layers:
                    fn(L)
                torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(R):
                for L in layers:
                    fn(L)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (R * len(layers))

        us = timed(lambda L: marca.mar_cache_attn_fwd(L["q_a"], L["k_a"], L["v_a"], L["k_cache"],
                                                      L["v_cache"], L["cached"], Nc=cfg.Nc,
                                                      out=L["out"]))
        nbytes = attn_bytes(cfg.B, cfg.H, cfg.A, cfg.Nc, cfg.D, 4 if cfg.dtype == "f32" else 2)
        gbs = nbytes / (us * 1e-6) / 1e9
        entry = {"sequences": cfg.B, "heads": cfg.H, "tokens": cfg.N, "active": cfg.A,
                 "cached": cfg.Nc, "attn_us_per_call": us, "attn_gbs": gbs,
                 "attn_frac_hbm": gbs / PEAK_HBM_GBS, "attn_bytes_per_call": nbytes,
                 "attn_tflops": 4 * cfg.B * cfg.H * cfg.A * (cfg.A + cfg.Nc) * cfg.D / us / 1e6}
        if name in ("mar_b", "mar_h"):
            # the floor of the call's access pattern (mar_bench_attn_pattern:
            # the same loads and stores, no arithmetic)
            from cache_aware_attention_amd import _bench_lib
            entry["attn_pattern_us"] = timed(lambda L: _bench_lib.mar_bench_attn_pattern(
                L["q_a"], L["k_a"], L["v_a"], L["k_cache"], L["v_cache"], L["cached"], cfg.Nc,
                L["out"]))
        if name == "highres":
            # the same kernel's floors (mar_bench_cached_floor): its
            # arithmetic alone and its memory operations alone
            from cache_aware_attention_amd import _bench_lib
            for key, mode in (("attn_arith_only_us", _bench_lib.MAR_BENCH_FLOOR_ARITH),
                              ("attn_memory_only_us", _bench_lib.MAR_BENCH_FLOOR_MEMORY)):
                entry[key] = timed(lambda L, mode=mode: _bench_lib.mar_bench_cached_floor(
                    L["q_a"], L["k_a"], L["v_a"], L["k_cache"], L["v_cache"], L["cached"],
                    L["out"], mode, Nc=cfg.Nc))
            full = torch.empty_like(layers[0]["k_cache"])
            flops = 4 * cfg.B * cfg.H * cfg.N * cfg.N * cfg.D
            # the queries: the K of the layer three away (no tensor is read
            # twice in a call or by two consecutive calls)
            qof = {id(L): layers[(i + 3) % len(layers)]["k_cache"] for i, L in enumerate(layers)}
            f_us = timed(lambda L: marca.mar_cache_attn_fwd(qof[id(L)], L["k_cache"], L["v_cache"],
                                                            L["k_cache"], L["v_cache"], None, Nc=0,
                                                            out=full))
            entry["full_attn_us_per_call"] = f_us
            entry["full_attn_tflops"] = flops / f_us / 1e6
            entry["full_attn_roofline"] = roofline_for(flops, 4 * cfg.B * cfg.H * cfg.N * cfg.D * 2,
                                                       f_us * 1e-6)
            # the same kernel's floors at this length (mar_bench_dense_floor)
            for key, mode in (("full_attn_arith_only_us", _bench_lib.MAR_BENCH_FLOOR_ARITH),
                              ("full_attn_memory_only_us", _bench_lib.MAR_BENCH_FLOOR_MEMORY)):
                entry[key] = timed(lambda L, mode=mode: _bench_lib.mar_bench_dense_floor(
                    qof[id(L)], L["k_cache"], L["v_cache"], full, mode))
            # refresh step: each layer's caches take the rows of the layer two
            # away as fresh K/V; the queries come from the layer four away
            nxt = {id(L): (layers[(i + 2) % len(layers)], layers[(i + 4) % len(layers)])
                   for i, L in enumerate(layers)}
            # the token gate at this shape (W = 1024, C5's gated layers)
            from mar_workloads import device_gate_features
            gx, gy, _ = device_gate_features(cfg.B, cfg.N, 1024, seed=cfg.seed, device=dev)
            g_us = timed(lambda L: marca.mar_cos_gate(gx, gy, 0.95))
            g_bytes = 2 * cfg.B * cfg.N * 1024 * 2 + cfg.B * cfg.N * 9
            entry["gate_us_per_call"] = g_us
            entry["gate_gbs"] = g_bytes / (g_us * 1e-6) / 1e9
            gl = {k: torch.empty((cfg.B, cfg.N), dtype=t, device=dev) for k, t in
                  (("cos", torch.float32), ("reuse", torch.uint8), ("cidx", torch.int32),
                   ("ridx", torch.int32))}
            gl["clen"], gl["rlen"] = (torch.empty((cfg.B,), dtype=torch.int32, device=dev)
                                      for _ in range(2))
            marca.mar_cos_gate(gx, gy, 0.95, cos_out=gl["cos"], reuse_mask=gl["reuse"],
                               compute_idx=gl["cidx"], compute_len=gl["clen"],
                               reuse_idx=gl["ridx"], reuse_len=gl["rlen"])
            torch.cuda.synchronize()
            del gx, gy
            entry["refresh_us_per_call"] = timed(
                lambda L: marca.mar_cache_attn_fwd_update(
                    nxt[id(L)][1]["k_cache"], nxt[id(L)][0]["k_cache"], nxt[id(L)][0]["v_cache"],
                    L["k_cache"], L["v_cache"], None, None, Nc=0, out=full))
            entry["gated_layer"] = gated_layer(marca, _bench_lib, cfg, layers, gl, dev, timed)
        res[name] = entry
        del layers
        torch.cuda.empty_cache()
    return res


def gated_layer(marca, bench_lib, cfg, layers, gl, dev, timed):
    """One gated layer of the high-res decode on each of the layers' caches:
    each sequence's recomputed tokens (the gate's compute list for seeded
    features at 84% reuse) attend over their fresh K/V and the cached K/V of
    the reused tokens, whose cache rows they replace in the same pass
    (mar_cache_attn_fwd_ragged_update), and the same kernel's floors."""
    import torch

    from mar_workloads import device_normal
    a = gl["clen"].long()
    cap = int(a.max())
    B, H, N, D = cfg.B, cfg.H, cfg.N, cfg.D
    x = {id(L): [device_normal((B, H, cap, D), 7700 + 3 * i + j, dev, torch.bfloat16)
                 for j in range(3)] + [torch.empty((B, H, cap, D), dtype=torch.bfloat16, device=dev)]
         for i, L in enumerate(layers)}
    torch.cuda.synchronize()

    def call(L, mode=None):
        q, k, v, o = x[id(L)]
        if mode is None:
            marca.mar_cache_attn_fwd_ragged_update(q, k, v, L["k_cache"], L["v_cache"], gl["ridx"],
                                                   gl["cidx"], gl["clen"], gl["rlen"], out=o)
        else:
            bench_lib.mar_bench_cached_floor(q, k, v, L["k_cache"], L["v_cache"], gl["ridx"], o,
                                             mode, active_idx=gl["cidx"], a_len=gl["clen"],
                                             c_len=gl["rlen"])

    us = timed(call)
    nbytes = ragged_update_bytes(H, N, D, a.tolist())
    gbs = nbytes / (us * 1e-6) / 1e9
    res = {"what": "mar_cache_attn_fwd_ragged_update at the high-res gated layers' counts; "
                   "floors as for the full attention (mar_bench_cached_floor)",
           "recomputed_mean": float(a.float().mean()), "recomputed_capacity": cap,
           "us_per_call": us, "bytes_per_call": nbytes, "gbs": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
           "tflops": 4 * H * D * N * float(a.sum()) / us / 1e6,
           "arith_only_us": timed(lambda L: call(L, bench_lib.MAR_BENCH_FLOOR_ARITH)),
           "memory_only_us": timed(lambda L: call(L, bench_lib.MAR_BENCH_FLOOR_MEMORY))}
    del x
    return res


C5_ROUNDS = 3
# the gated layers' attention and cache update in one call (the default), or
# as the ragged attention followed by the scatter (--c5-separate-update)
C5_FUSED_UPDATE = [True]


def c5_decode(marca, dev, stream, rounds=C5_ROUNDS, modes=("cache", "none", "cache+cond")):
    """The high-res configuration's whole 64-step decode of the attention path
    at full size: 64 sequences (32 images x 2 CFG), 16 heads, 1088 tokens (64
    prefix + 1024 image), 32 layers, active budget 128, a refresh every third
    step, and LazyMAR's token gate on layers 4-32 (1024-wide features,
    threshold 0.95, seeded 84% reuse).  A cached step runs: layer 1 full
    attention; layer 2 full attention, then the refresh scores + top-K over
    the same K (mar_refresh_topk: 1088 tokens is past the single-pass scores
    kernel);
    layer 3 the fused cache-aware attention + cache update of its 128 active
    rows; layers 4-32 the gate (which also lists each sequence's reused
    positions), and the ragged attention of each sequence's recomputed
    tokens over their fresh K/V and the cached K/V of its reused tokens,
    fused with the cache update of the recomputed rows
    (mar_cache_attn_fwd_ragged_update; --c5-separate-update runs the ragged
    attention and then the scatter instead); the CFG residual reuse.  A refresh step runs full attention in every layer, layers 3-32
    rewriting their caches in the same call, and stores the CFG residual.
    Modes as for MAR-L: no caches (full attention everywhere), the caches,
    and the caches + condition cache (the steps between refreshes compute the
    conditional half of the batch only).  Every layer has its own caches,
    gate features and recomputed-row Q/K/V; the fresh Q/K/V of a
    full-attention call are other layers' caches a third and two thirds of
    the stack away, so no tensor is read by two consecutive calls.  The gate
    features do not change between steps (their upkeep is the model's), so
    each layer recomputes the same tokens at every step."""
    import torch

    from mar_workloads import (CONFIGS, cfg_outputs, cosine_counts, device_gate_features,
                               device_normal, generation_order)
    cfg = CONFIGS["highres"]
    B, H, N, D, L = cfg.B, cfg.H, cfg.N, cfg.D, cfg.layers
    n_ca = L - 2                   # cache-aware layers 3..32 (index 0 is layer 3)
    n_gated = n_ca - 1             # layers 4..32 (index 1..)
    bf = torch.bfloat16
    t_setup = time.perf_counter()
    kc = [device_normal((B, H, N, D), 8000 + 2 * i, dev, bf) for i in range(n_ca)]
    vc = [device_normal((B, H, N, D), 8001 + 2 * i, dev, bf) for i in range(n_ca)]
    counts = cosine_counts(cfg.n_img, cfg.steps)
    plans = [marca.mar_plan_step(counts, t, N, cfg.budget) for t in range(cfg.steps)]
    order = torch.from_numpy(generation_order(cfg)).to(dev)
    # per step: the G then P list of the top-K and the generating queries of layer 2
    gp = {}
    qgen = {}
    for t, p in enumerate(plans):
        if p.refresh:
            continue
        gp[t] = order[:, p.prev_begin:p.gen_begin + p.n_gen].contiguous()
        if p.n_gen not in qgen:
            qgen[p.n_gen] = device_normal((B, H, p.n_gen, D), 8900 + p.n_gen, dev, bf)
    A3 = cfg.budget
    q3, k3, v3 = (device_normal((B, H, A3, D), 8800 + i, dev, bf) for i in range(3))
    ws = torch.empty((marca.mar_refresh_topk_workspace(B, H, N) // 4,), dtype=torch.float32,
                     device=dev)
    sel = {"scores": torch.empty((B, N), dtype=torch.float32, device=dev),
           "active": torch.empty((B, A3), dtype=torch.int32, device=dev),
           "cached": torch.empty((B, N - A3), dtype=torch.int32, device=dev),
           "clen": torch.empty((B,), dtype=torch.int32, device=dev)}
    gate_out = {"cos": torch.empty((B, N), dtype=torch.float32, device=dev),
                "reuse": torch.empty((B, N), dtype=torch.uint8, device=dev),
                "cidx": torch.empty((B, N), dtype=torch.int32, device=dev),
                "clen": torch.empty((B,), dtype=torch.int32, device=dev),
                "ridx": torch.empty((B, N), dtype=torch.int32, device=dev),
                "rlen": torch.empty((B,), dtype=torch.int32, device=dev)}
    gx, gy, qc, kcn, vcn, acap = [None], [None], [None], [None], [None], [0]
    for i in range(1, n_ca):
        x_cur, x_cached, _ = device_gate_features(B, N, cfg.W, seed=cfg.seed + 17 * i, device=dev)
        gx.append(x_cur)
        gy.append(x_cached)
        marca.mar_cos_gate(x_cur, x_cached, cfg.tau, compute_len=gate_out["clen"])
        cap = int(gate_out["clen"].max())  # the recomputed rows' capacity (same every step)
        acap.append(cap)
        qc.append(device_normal((B, H, cap, D), 9000 + 3 * i, dev, bf))
        kcn.append(device_normal((B, H, cap, D), 9001 + 3 * i, dev, bf))
        vcn.append(device_normal((B, H, cap, D), 9002 + 3 * i, dev, bf))
    c0, u0, c1, _ = cfg_outputs(cfg.B_img, cfg.n_img, 16, seed=cfg.seed)
    cond = torch.from_numpy(c1).to(dev)
    uncond = torch.from_numpy(u0).to(dev)
    residual = torch.from_numpy(c0 - u0).to(dev)
    uncond_out = torch.empty_like(cond)
    full_out = torch.empty((B, H, N, D), dtype=bf, device=dev)
    out3 = torch.empty((B, H, A3, D), dtype=bf, device=dev)
    outc = [None] + [torch.empty_like(qc[i]) for i in range(1, n_ca)]
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    P = marca.prepare
    prep = {}
    half = [B]

    def run(key, fn, *a, **kw):
        """fn(*a, **kw) marshalled once per (batch size, key), then replayed."""
        k = (half[0],) + key
        if k not in prep:
            nb = half[0]
            a = [t[:nb] if isinstance(t, torch.Tensor) and t.shape[0] == B else t for t in a]
            kw = {n: (t[:nb] if isinstance(t, torch.Tensor) and t.shape[0] == B else t)
                  for n, t in kw.items()}
            prep[k] = P(fn, *a, **kw)
        prep[k]()

    third = n_ca // 3

    def full(l):  # full attention of layer l (0..31): K/V of cache l mod 30, Q two thirds away
        i = l % n_ca
        run(("full", l), marca.mar_cache_attn_fwd, kc[(i + 2 * third) % n_ca], kc[i], vc[i],
            kc[i], vc[i], None, Nc=0, out=full_out, stream=stream)

    def refresh(i):  # cache-aware layer i on a refresh step: fresh K/V a third away
        j, k = (i + third) % n_ca, (i + 2 * third) % n_ca
        run(("refresh", i), marca.mar_cache_attn_fwd_update, kc[k], kc[j], vc[j], kc[i], vc[i],
            None, None, Nc=0, out=full_out, stream=stream)

    def cached_step(t):
        p = plans[t]
        full(0)
        full(1)
        run(("topk", t), marca.mar_refresh_topk, qgen[p.n_gen], kc[1], gp[t],
            p.n_prev + p.n_gen, p.n_refresh, scores=sel["scores"], active_idx=sel["active"],
            cached_idx=sel["cached"], cached_len=sel["clen"], workspace=ws, stream=stream)
        run(("fused",), marca.mar_cache_attn_fwd_update, q3, k3, v3, kc[0], vc[0], sel["cached"],
            sel["active"], Nc=N - A3, out=out3, stream=stream)
        for i in range(1, n_ca):
            run(("gate", i), marca.mar_cos_gate, gx[i], gy[i], cfg.tau, cos_out=gate_out["cos"],
                reuse_mask=gate_out["reuse"], compute_idx=gate_out["cidx"],
                compute_len=gate_out["clen"], reuse_idx=gate_out["ridx"],
                reuse_len=gate_out["rlen"], stream=stream)
            if C5_FUSED_UPDATE[0]:
                run(("ragged_update", i), marca.mar_cache_attn_fwd_ragged_update, qc[i], kcn[i],
                    vcn[i], kc[i], vc[i], gate_out["ridx"], gate_out["cidx"], gate_out["clen"],
                    gate_out["rlen"], out=outc[i], stream=stream)
            else:
                run(("ragged", i), marca.mar_cache_attn_fwd_ragged, qc[i], kcn[i], vcn[i], kc[i],
                    vc[i], gate_out["ridx"], gate_out["clen"], gate_out["rlen"], out=outc[i],
                    stream=stream)
                run(("scatter", i), marca.mar_kv_scatter_refresh, kc[i], vc[i], kcn[i], vcn[i],
                    gate_out["cidx"], stream=stream)
        run(("cfg_reuse",), marca.mar_cfg_residual, cond, residual=residual,
            mode=marca.MAR_CFG_REUSE, uncond_out=uncond_out, stream=stream)

    def decode(mode):
        for t, p in enumerate(plans):
            if mode == "none":
                for l in range(L):
                    full(l)
                continue
            if p.refresh:
                full(0)
                full(1)
                for i in range(n_ca):
                    refresh(i)
                run(("cfg_store",), marca.mar_cfg_residual, cond, uncond, residual=residual,
                    mode=marca.MAR_CFG_STORE, stream=stream)
                continue
            if mode == "cache+cond":
                half[0] = B // 2
            cached_step(t)
            half[0] = B

    samples = {m: [] for m in modes}
    for m in modes:
        decode(m)
    torch.cuda.synchronize()
    for r in range(rounds):
        for j in range(len(modes)):
            m = modes[(j + r) % len(modes)]
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            decode(m)
            e1.record(stream)
            torch.cuda.synchronize()
            samples[m].append(e0.elapsed_time(e1))
    med = {m: sorted(v)[len(v) // 2] for m, v in samples.items()}
    ms = lambda m: med.get(m)
    ratio = lambda a, b: (med[a] / med[b]) if a in med and b in med else None
    res = {
        "what": " ".join(c5_decode.__doc__.split()),
        "sequences": B, "heads": H, "tokens": N, "layers": L, "budget": cfg.budget,
        "gate_width": cfg.W, "gated_layers": n_gated, "steps": cfg.steps,
        "refresh_steps": sum(p.refresh for p in plans),
        "recomputed_rows_capacity": acap[1:],
        "gated_layer_update": "fused" if C5_FUSED_UPDATE[0] else "separate scatter",
        "timing": f"median of {rounds} interleaved runs per mode",
        "samples_ms": samples,
        "ms": ms("cache"), "ms_no_cache": ms("none"), "ms_cond_cache": ms("cache+cond"),
        "speedup": ratio("none", "cache"),
        "speedup_cond_cache": ratio("none", "cache+cond"),
        "setup_s": setup_s,
    }
    del kc, vc, gx, gy, qc, kcn, vcn, prep
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the whole-decode timing (for counter runs)")
    ap.add_argument("--c5-only", action="store_true",
                    help="only the full-size high-res 64-step decode (one JSON object)")
    ap.add_argument("--c5-modes", default="cache,none,cache+cond",
                    help="with --c5-only: the decode modes to run (comma-separated)")
    ap.add_argument("--c5-separate-update", action="store_true",
                    help="with --c5-only: the gated layers' cache update as a separate scatter")
    ap.add_argument("--locality-only", action="store_true",
                    help="only the locality comparison's kernels, a fixed sequence (counter runs)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run the plain copy kernel (counter calibration)")
    ap.add_argument("--configs-only", action="store_true",
                    help="only the other configurations' calls (one JSON object; counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence with no collective; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import cache_aware_attention_amd as marca
    from mar_workloads import CONFIGS, cosine_counts

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = CONFIGS["mar_l"]

    if args.c5_only:
        C5_FUSED_UPDATE[0] = not args.c5_separate_update
        modes = tuple(m for m in args.c5_modes.split(",") if m)
        if not modes or any(m not in ("cache", "none", "cache+cond") for m in modes):
            print(f"bench: unknown --c5-modes {args.c5_modes!r}", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(c5_decode(marca, dev, torch.cuda.current_stream(), modes=modes)))
        return

    if args.locality_only:
        # Per split, in this order: 3 passes of the cache-aware attention over
        # its layers, then 3 of the concatenation, then 3 of the attention over
        # the concatenated rows; one line of JSON with the dispatch order.
        stream = torch.cuda.current_stream()
        order = []
        for A in LOCALITY_SPLITS:
            _, layers = locality_inputs(marca, dev, A, stream)
            for key, name in (("p_ca", "cache_aware"), ("p_cat", "concat"),
                              ("p_std", "attention_on_concat")):
                for _ in range(3):
                    for x in layers:
                        x[key]()
                order.append({"active": A, "variant": name, "launches": 3 * len(layers)})
            torch.cuda.synchronize()
            del layers
            torch.cuda.empty_cache()
        print(json.dumps({"dispatch_order": order}))
        return

    if args.configs_only:
        print(json.dumps(other_configs(marca, dev, torch.cuda.current_stream())))
        return

    if args.copy_only:
        # plain copy of a known size through the full-refresh kernel: 2 x 256 MiB read,
        # 2 x 256 MiB written per launch
        n = 256 * 1024 * 1024 // 2
        a = torch.empty(n, dtype=torch.bfloat16, device=dev).view(1, 1, n // 64, 64)
        b = torch.empty_like(a); c = torch.empty_like(a); d = torch.empty_like(a)
        for _ in range(5):
            marca.mar_kv_scatter_refresh(a, b, c, d, None)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": 2 * n * 2,
                          "copy_bytes_written_per_launch": 2 * n * 2}))
        return

    print(f"bench: building MAR-L inputs ({cfg.layers - 2} cache-aware layers)", file=sys.stderr,
          flush=True)
    x = build_inputs(cfg, dev)
    # layer 2 in two passes needs the generating rows of each layer's queries
    # (the K of the layer half the stack away stands in for layer l's
    # queries, as in full_attn below) as their own tensor
    n_layers = cfg.layers - 2
    gen_pos = x["gp"][:, cfg.n_prev:cfg.n_prev + cfg.n_gen].long()
    gidx = gen_pos[:, None, :, None].expand(cfg.B, cfg.H, cfg.n_gen, cfg.D)
    for l in range(n_layers):
        Lq = x["layers"][(l + n_layers // 2) % n_layers]["k_cache"]
        x["layers"][l]["q_gen2"] = torch.gather(Lq, 2, gidx).contiguous()
    torch.cuda.synchronize()
    counts = [cfg.n_gen] * (cfg.steps)
    counts[0] = 0
    # the whole decode follows the cosine masking schedule over the 256 image tokens
    decode_counts = cosine_counts(cfg.n_img, cfg.steps)
    step_t = 4  # a non-refresh step (4 % 3 != 0) with 16 previous + 16 generating tokens
    n_ca = cfg.layers - 2

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # The K/V scatters run on a second stream (default priority).  Layer l's
    # scatter writes the active rows of layer l's cache, which no later layer
    # reads, so it only has to wait until layer l's fresh K/V exist (layer
    # l - 1 done); the step ends by joining the two streams.
    side = torch.cuda.Stream()
    layer_done = [torch.cuda.Event() for _ in range(cfg.layers)]
    side_done = torch.cuda.Event()
    # The sequences the step functions below run on: the whole batch, or (on a
    # condition-cache step of the decode) its conditional half.  Every call of
    # the timed loops is marshalled once (marca.prepare: device pointers,
    # sizes and stream fixed), so the host issues a launch in a few
    # microseconds and stays ahead of the GPU.
    X = [x]
    x_cond = seq_view(x, cfg.B_img)
    half = lambda: X[0] is x_cond
    P = marca.prepare
    prep = {}

    def prepared(key, fn, *a, **kw):
        """The prepared form of fn(*a, **kw) for the current batch half."""
        k = (half(),) + key
        if k not in prep:
            prep[k] = P(fn, *a, **kw)
        return prep[k]

    def topk(plan):
        x = X[0]
        prepared(("topk", plan.n_prev + plan.n_gen, plan.n_refresh), marca.mar_refresh_topk,
                 x["q_gen"], x["k_full"], x["gp"], plan.n_prev + plan.n_gen, plan.n_refresh,
                 scores=x["scores"], active_idx=x["active_idx"], cached_idx=x["cached_idx"],
                 cached_len=x["cached_len"], workspace=x["workspace"], stream=stream)()

    def attn(l, plan):
        x = X[0]
        L = x["layers"][l]
        prepared(("attn", l, plan.n_cached), marca.mar_cache_attn_fwd, L["q_a"], L["k_a"],
                 L["v_a"], L["k_cache"], L["v_cache"], x["cached_idx"], Nc=plan.n_cached,
                 out=L["out"], stream=stream)()

    def scatter(l, on=None):
        x = X[0]
        L = x["layers"][l]
        prepared(("scatter", l, on is not None), marca.mar_kv_scatter_refresh, L["k_cache"],
                 L["v_cache"], L["k_a"], L["v_a"], x["active_idx"],
                 stream=stream if on is None else on)()

    def cached_layers(plan):
        """Layers 3-32 of a cached step: attention on the main stream, each
        layer's scatter on the side stream once the previous layer is done."""
        layer_done[0].record(stream)
        for l in range(n_ca):
            side.wait_event(layer_done[l])
            scatter(l, on=side)
            attn(l, plan)
            layer_done[l + 1].record(stream)
        side_done.record(side)
        stream.wait_event(side_done)

    def fused(l, plan):
        x = X[0]
        L = x["layers"][l]
        prepared(("fused", l, plan.n_cached), marca.mar_cache_attn_fwd_update, L["q_a"], L["k_a"],
                 L["v_a"], L["k_cache"], L["v_cache"], x["cached_idx"], x["active_idx"],
                 Nc=plan.n_cached, out=L["out"], stream=stream)()

    def full_attn(l):
        """A full-attention layer (layers 1-2 of every step, every layer of a
        refresh step): all N tokens active, no cached rows.  Layer l's stored
        K/V stand in for its fresh K/V and the K of the layer half the stack
        away for its Q, so that no tensor is read by two consecutive calls
        (consecutive layers' working sets would otherwise share one in the
        last-level cache)."""
        x = X[0]
        L, Lq = x["layers"][l], x["layers"][(l + n_ca // 2) % n_ca]
        prepared(("full", l), marca.mar_cache_attn_fwd, Lq["k_cache"], L["k_cache"], L["v_cache"],
                 L["k_cache"], L["v_cache"], None, Nc=0, out=x["full_out"], stream=stream)()

    def layer2_separate(l, plan):
        """Layer 2 of a cached step as two passes over its K: the full
        attention (layer l's buffers), then the refresh scores + top-K of
        mar_refresh_topk on the generating rows of the same queries."""
        x = X[0]
        L = x["layers"][l]
        full_attn(l)
        prepared(("l2topk", l, plan.n_prev + plan.n_gen, plan.n_refresh), marca.mar_refresh_topk,
                 L["q_gen2"], L["k_cache"], x["gp"], plan.n_prev + plan.n_gen, plan.n_refresh,
                 scores=x["scores"], active_idx=x["active_idx"], cached_idx=x["cached_idx"],
                 cached_len=x["cached_len"], workspace=x["workspace"], stream=stream)()

    def layer2_fused(l, plan):
        """Layer 2 of a cached step in one pass over its K: the full attention
        that also writes the generating queries' per-head probability sums,
        then the selection from them."""
        x = X[0]
        L, Lq = x["layers"][l], x["layers"][(l + n_ca // 2) % n_ca]
        gen = x["gp"][:, plan.n_prev:plan.n_prev + plan.n_gen]
        prepared(("l2scores", l, plan.n_prev, plan.n_gen), marca.mar_cache_attn_fwd_scores,
                 Lq["k_cache"], L["k_cache"], L["v_cache"], gen, plan.n_gen,
                 partials=x["partials"], out=x["full_out"], stream=stream)()
        prepared(("l2select", plan.n_prev + plan.n_gen, plan.n_refresh, plan.n_gen),
                 marca.mar_refresh_select, x["partials"], x["gp"], plan.n_prev + plan.n_gen,
                 plan.n_refresh, plan.n_gen, scores=x["scores"], active_idx=x["active_idx"],
                 cached_idx=x["cached_idx"], cached_len=x["cached_len"], stream=stream)()

    def cfg_reuse():
        prepared(("cfg_reuse",), marca.mar_cfg_residual, x["cond"], residual=x["residual"],
                 mode=marca.MAR_CFG_REUSE, uncond_out=x["uncond_out"], stream=stream)()

    def cfg_store():
        prepared(("cfg_store",), marca.mar_cfg_residual, x["cond"], x["uncond_out"],
                 residual=x["residual"], mode=marca.MAR_CFG_STORE, stream=stream)()

    def gate():
        x = X[0]
        prepared(("gate",), marca.mar_cos_gate, x["gate_x"], x["gate_y"], 0.95, cos_out=x["cos"],
                 reuse_mask=x["reuse"], compute_idx=x["cidx"], compute_len=x["clen"],
                 stream=stream)()

    def plan_step():
        plan = marca.mar_plan_step(counts, step_t, cfg.N, cfg.budget)
        assert not plan.refresh and plan.n_active == cfg.A and plan.n_cached == cfg.Nc
        return plan

    def one_step():
        """One decode step in model order: top-K at layer 2, then per cache-aware
        layer its attention and the scatter of its fresh rows (overlapped on the
        side stream), then CFG + gate."""
        plan = plan_step()
        topk(plan)
        cached_layers(plan)
        cfg_reuse()
        gate()

    def one_step_fused():
        """The same step with each layer's attention and cache update in one kernel."""
        plan = plan_step()
        topk(plan)
        for l in range(n_ca):
            fused(l, plan)
        cfg_reuse()
        gate()

    def full_refresh(l):
        """A refresh step of cache-aware layer l: full attention over all N tokens
        and the rewrite of every row of the layer's cache with the fresh K/V, in
        one call (the stored K/V of the layer a third of the stack away stand in
        for the fresh K/V, the K of the layer two thirds away for Q: no tensor
        is read by two consecutive calls)."""
        x = X[0]
        L, Ln, Lq = (x["layers"][(l + i * (n_ca // 3)) % n_ca] for i in range(3))
        prepared(("refresh", l), marca.mar_cache_attn_fwd_update, Lq["k_cache"], Ln["k_cache"],
                 Ln["v_cache"], L["k_cache"], L["v_cache"], None, None, Nc=0, out=x["full_out"],
                 stream=stream)()

    def decode(use_cache, cond_cache=False):
        """A whole 64-step decode of the attention path.  With the cache: on a
        refresh step (t mod 3 = 0) every layer runs full attention and rewrites
        its cache, and the CFG residual is stored; on the other steps layers 1-2
        run full attention and layers 3-32 the fused cached layers of the step
        above.  With the condition cache as well, those other steps compute the
        conditional branch only (half the sequences) and take the unconditional
        output from the stored residual.  On a cached step layer 2's attention
        also yields the refresh scores (mar_cache_attn_fwd_scores) and the
        selection reads them (mar_refresh_select).  Without the cache every layer of every step runs
        full attention."""
        for t in range(cfg.steps):
            if not use_cache:
                for l in range(cfg.layers):
                    full_attn(l % n_ca)
                continue
            plan = plans[t]
            if plan.refresh:
                full_attn(0)
                full_attn(1)
                for l in range(n_ca):
                    full_refresh(l)
                cfg_store()
                continue
            if cond_cache:
                X[0] = x_cond
            full_attn(0)
            layer2_fused(1, plan)
            for l in range(n_ca):
                fused(l, plan)
            cfg_reuse()
            gate()
            X[0] = x

    plans = [marca.mar_plan_step(decode_counts, t, cfg.N, cfg.budget) for t in range(cfg.steps)]

    from cache_aware_attention_amd import _bench_lib

    def pattern(l, write_out):
        """The attention's memory operations without its arithmetic (its
        access-pattern floor), on layer l's buffers."""
        x = X[0]
        L = x["layers"][l]
        prepared(("pattern", l, write_out), _bench_lib.mar_bench_attn_pattern, L["q_a"], L["k_a"],
                 L["v_a"], L["k_cache"], L["v_cache"], x["cached_idx"], cfg.Nc, L["out"],
                 write_out=write_out, stream=stream)()

    def full_floor(l, mode):
        """The full-attention kernel on layer l's buffers (as full_attn) in a
        measurement mode: its arithmetic alone or its memory operations alone."""
        x = X[0]
        L, Lq = x["layers"][l], x["layers"][(l + n_ca // 2) % n_ca]
        prepared(("full_floor", l, mode), _bench_lib.mar_bench_dense_floor, Lq["k_cache"],
                 L["k_cache"], L["v_cache"], x["full_out"], mode, stream=stream)()

    def refresh_floor(l, mode):
        """The refresh-step layer on full_refresh's buffers in a measurement mode."""
        x = X[0]
        L, Ln, Lq = (x["layers"][(l + i * (n_ca // 3)) % n_ca] for i in range(3))
        prepared(("refresh_floor", l, mode), _bench_lib.mar_bench_dense_floor, Lq["k_cache"],
                 Ln["k_cache"], Ln["v_cache"], x["full_out"], mode, k_cache=L["k_cache"],
                 v_cache=L["v_cache"], stream=stream)()

    def timed_kernels():
        """The same launches as one step, grouped by kernel so that one pair of HIP
        events brackets each group of back-to-back launches (an event pair around
        every single launch adds its own overhead to the measured time)."""
        plan = plan_step()
        spans = {}
        def span(name, fn, n):
            e0 = ev(); e0.record(stream)
            fn()
            e1 = ev(); e1.record(stream)
            spans[name] = (e0, e1, n)
        span("topk", lambda: topk(plan), 1)
        span("attn", lambda: [attn(l, plan) for l in range(n_ca)], n_ca)
        span("scatter", lambda: [scatter(l) for l in range(n_ca)], n_ca)
        span("attn_update", lambda: [fused(l, plan) for l in range(n_ca)], n_ca)
        span("cfg", cfg_reuse, 1)
        span("gate", gate, 1)
        span("full_attn", lambda: [full_attn(l) for l in range(n_ca)], n_ca)
        span("full_refresh", lambda: [full_refresh(l) for l in range(n_ca)], n_ca)
        span("full_arith_only", lambda: [full_floor(l, _bench_lib.MAR_BENCH_FLOOR_ARITH)
                                         for l in range(n_ca)], n_ca)
        span("full_memory_only", lambda: [full_floor(l, _bench_lib.MAR_BENCH_FLOOR_MEMORY)
                                          for l in range(n_ca)], n_ca)
        span("refresh_arith_only", lambda: [refresh_floor(l, _bench_lib.MAR_BENCH_FLOOR_ARITH)
                                            for l in range(n_ca)], n_ca)
        span("refresh_memory_only", lambda: [refresh_floor(l, _bench_lib.MAR_BENCH_FLOOR_MEMORY)
                                             for l in range(n_ca)], n_ca)
        span("attn_pattern", lambda: [pattern(l, True) for l in range(n_ca)], n_ca)
        span("attn_pattern_reads", lambda: [pattern(l, False) for l in range(n_ca)], n_ca)
        span("layer2_separate", lambda: [layer2_separate(l, plan) for l in range(n_ca)], n_ca)
        span("layer2_fused", lambda: [layer2_fused(l, plan) for l in range(n_ca)], n_ca)
        return spans

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        one_step_fused()
    torch.cuda.synchronize()

    # Timed region 1: whole steps (fused attention + cache update), no
    # per-kernel events.
    print("bench: timing steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    s0, s1 = ev(), ev()
    t0 = time.perf_counter()
    s0.record(stream)
    for _ in range(args.steps):
        one_step_fused()
    s1.record(stream)
    issue = time.perf_counter() - t0  # host time to issue the steps (no wait)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = s0.elapsed_time(s1) / args.steps

    # Timed region 1b: whole steps with attention and scatter as separate
    # kernels (the scatters on the side stream).
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    f0, f1 = ev(), ev()
    f0.record(stream)
    for _ in range(args.steps):
        one_step()
    f1.record(stream)
    torch.cuda.synchronize()
    ms_per_step_unfused = f0.elapsed_time(f1) / args.steps

    # Timed region 2: the same launches, grouped per kernel, HIP events per group.
    # Timed before the decodes, whose second of heavy load slows later groups.
    # One untimed pass first: the first span of the first pass would otherwise
    # take in the host's delay before its first launch.
    # At most 30 passes (900 launches of each kernel): over longer runs of
    # these back-to-back heavy groups the later ones slow down (the refresh
    # layers by 10-15%), which is the chip's sustained-load behaviour, not
    # the kernels'.
    timed_kernels()
    torch.cuda.synchronize()
    groups = [timed_kernels() for _ in range(min(args.steps, 30))]
    torch.cuda.synchronize()
    avg_us = {k: 1e3 * sum(g[k][0].elapsed_time(g[k][1]) for g in groups)
              / sum(g[k][2] for g in groups) for k in groups[0]}
    per_pass = sorted(1e3 * g["attn"][0].elapsed_time(g["attn"][1]) / g["attn"][2] for g in groups)
    attn_median_us = per_pass[len(per_pass) // 2]

    # Timed region 3: whole decodes, with and without the caches.  Each mode
    # once untimed, then DECODE_ROUNDS timed rounds that run every mode in a
    # rotated order (so no mode always follows the heavy no-cache decode);
    # the median per mode is reported, with every sample.
    modes = () if args.no_decode else ("cache", "none", "cache+cond")
    decode_samples = {m: [] for m in modes}

    def run_decode(mode):
        decode(mode != "none", cond_cache=mode == "cache+cond")

    for mode in modes:
        run_decode(mode)
    torch.cuda.synchronize()
    for r in range(DECODE_ROUNDS if modes else 0):
        for i in range(len(modes)):
            mode = modes[(i + r) % len(modes)]
            d0, d1 = ev(), ev()
            d0.record(stream)
            run_decode(mode)
            d1.record(stream)
            torch.cuda.synchronize()
            decode_samples[mode].append(d0.elapsed_time(d1))
    decode_ms = {m: sorted(v)[len(v) // 2] for m, v in decode_samples.items()}
    n_refresh_steps = sum(marca.mar_plan_step(decode_counts, t, cfg.N, cfg.budget).refresh
                          for t in range(cfg.steps))


    tokens_per_step = cfg.B * cfg.A * n_ca
    bytes_call = attn_bytes(cfg.B, cfg.H, cfg.A, cfg.Nc, cfg.D)
    achieved = bytes_call / (avg_us["attn"] * 1e-6) / 1e9
    bytes_fused = fused_bytes(cfg.B, cfg.H, cfg.A, cfg.Nc, cfg.D)
    achieved_fused = bytes_fused / (avg_us["attn_update"] * 1e-6) / 1e9

    full_flops = 4 * cfg.B * cfg.H * cfg.N * cfg.N * cfg.D
    full_tflops = full_flops / (avg_us["full_attn"] * 1e-6) / 1e12
    full_bytes = 4 * cfg.B * cfg.H * cfg.N * cfg.D * 2

    copy_gbs = None
    try:  # achievable HBM: the plain full-refresh copy, layer i + 1's caches into layer i's
        Ls = x["layers"]
        e0, e1 = ev(), ev()
        e0.record(stream)
        for i in range(10):  # ten different pairs: no tensor is read or written twice
            marca.mar_kv_scatter_refresh(Ls[i]["k_cache"], Ls[i]["v_cache"], Ls[i + 1]["k_cache"],
                                         Ls[i + 1]["v_cache"], None)
        e1.record(stream)
        torch.cuda.synchronize()
        nbytes = 4 * Ls[0]["k_cache"].numel() * 2
        copy_gbs = nbytes / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    except Exception as exc:  # noqa: BLE001 - reported, not fatal
        print(f"bench: copy measurement failed: {exc}", file=sys.stderr)

    def optional(name, fn):
        # a leg outside the headline that raises is reported in its own field
        # (and on stderr) instead of taking the headline record down with it
        try:
            return fn()
        except Exception as exc:  # noqa: BLE001 - reported in the record
            print(f"bench: {name} failed: {exc!r}", file=sys.stderr, flush=True)
            return {"error": repr(exc)}

    configs = None if args.no_decode else optional(
        "configs", lambda: other_configs(marca, dev, stream))
    loc = None if args.no_decode else optional("locality", lambda: locality(marca, dev, stream))
    if not args.no_decode:
        print("bench: high-res 64-step decode", file=sys.stderr, flush=True)
    c5 = None if args.no_decode else optional("c5_decode", lambda: c5_decode(marca, dev, stream))

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: oracle CPU baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(x, cfg.Nc, cfg, args)

    line = headline_record(cfg, n_ca, args.steps, args.warmup, ms_per_step, achieved_fused,
                           load_traffic("fused"), cpu)
    line["roofline"].update({"kernel": "mar_cache_attn_fwd_update (attention + cache update)",
                             "bytes_per_call": bytes_fused,
                             "us_per_call": avg_us["attn_update"]})
    def hbm_rate(us, nbytes):
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"us_per_call": us, "bytes_per_call": nbytes, "gbs": gbs,
                "frac_hbm": gbs / PEAK_HBM_GBS}

    B_, H_, N_, D_ = cfg.B, cfg.H, cfg.N, cfg.D
    line.update({
        "kernel_us": avg_us,
        "step_kernels": {
            "what": "the step's other kernels against 8 TB/s, algorithmic bytes per call: the "
                    "top-K reads the generating queries and layer 2's K and writes the scores "
                    "and the partition, the scatter reads and writes the active rows, the gate "
                    "reads both feature sets and writes cosines, mask and list; the CFG residual "
                    "(about 3 MB) is reported in microseconds only",
            "topk": hbm_rate(avg_us["topk"], B_ * H_ * (cfg.n_gen + N_) * D_ * 2 + B_ * N_ * 5
                             + B_ * (cfg.K + cfg.Nc) * 4),
            "scatter": hbm_rate(avg_us["scatter"], 4 * B_ * H_ * cfg.A * D_ * 2),
            "gate": hbm_rate(avg_us["gate"], 2 * B_ * N_ * cfg.W * 2 + B_ * N_ * 9),
            "cfg_us_per_call": avg_us["cfg"]},
        "attention_roofline": {
            "what": "the cache-aware attention alone (mar_cache_attn_fwd), same layers",
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": load_traffic("attention"),
            "bytes_per_call": bytes_call, "us_per_call": avg_us["attn"]},
        "unfused_step": {
            "what": "the same step with mar_cache_attn_fwd + mar_kv_scatter_refresh (the "
                    "scatters on a second stream) in place of the fused kernel",
            "ms_per_step": ms_per_step_unfused,
            "value": tokens_per_step / (ms_per_step_unfused * 1e-3)},
        "full_attention": {
            "what": "mar_cache_attn_fwd with A = N and no cached rows (layers 1-2 of every "
                    "step, every layer of a refresh step), outside the step above",
            "us_per_call": avg_us["full_attn"],
            "refresh_us_per_call": avg_us["full_refresh"],
            "refresh_what": "the same layer on a refresh step: mar_cache_attn_fwd_update with no "
                            "active list (full attention and every cache row rewritten, one call)",
            "roofline": roofline_for(full_flops, full_bytes, avg_us["full_attn"] * 1e-6),
            "tflops": full_tflops,
            "refresh_roofline": roofline_for(full_flops, full_bytes + 2 * full_bytes // 4,
                                             avg_us["full_refresh"] * 1e-6),
            "floors": {
                "what": "the same kernel on the same layers in its measurement modes "
                        "(mar_bench_dense_floor): its arithmetic, LDS traffic and barriers "
                        "alone (no memory traffic) and its memory operations alone (no "
                        "per-chunk math); the layer cannot take less than the larger",
                "arith_only_us": avg_us["full_arith_only"],
                "memory_only_us": avg_us["full_memory_only"],
                "memory_only_gbs": full_bytes / (avg_us["full_memory_only"] * 1e-6) / 1e9,
                "refresh_arith_only_us": avg_us["refresh_arith_only"],
                "refresh_memory_only_us": avg_us["refresh_memory_only"],
                "refresh_memory_only_gbs": (full_bytes + 2 * full_bytes // 4)
                                           / (avg_us["refresh_memory_only"] * 1e-6) / 1e9}},
        "decode": None if args.no_decode else {
            "what": "one 64-step decode of the attention path (every layer's attention, cache "
                    "writes, top-K, CFG and gate; no projections or MLPs), with the cache "
                    "(refresh every 3rd step) and without it (full attention everywhere); "
                    "ms_cond_cache adds the condition cache: the steps between refreshes "
                    "compute the conditional half of the batch only",
            "steps": cfg.steps, "refresh_steps": n_refresh_steps, "layers": cfg.layers,
            "timing": f"median of {DECODE_ROUNDS} interleaved runs per mode",
            "samples_ms": decode_samples,
            "ms": decode_ms.get("cache"), "ms_no_cache": decode_ms.get("none"),
            "speedup": decode_ms.get("none", 0) / decode_ms.get("cache", 1),
            "ms_cond_cache": decode_ms.get("cache+cond"),
            "speedup_cond_cache": decode_ms.get("none", 0) / decode_ms.get("cache+cond", 1)},
        "configs": configs,
        "attn_pattern": {
            "what": "the attention's memory operations without its arithmetic "
                    "(mar_bench_attn_pattern): the floor of its access pattern, same buffers",
            "us_per_call": avg_us["attn_pattern"],
            "reads_only_us_per_call": avg_us["attn_pattern_reads"],
            "attn_over_pattern": avg_us["attn"] / avg_us["attn_pattern"]},
        "layer2": {
            "what": "layer 2 of a cached step (full attention over 320 tokens + the refresh "
                    "top-K): as the full attention then mar_refresh_topk (which reads K again), "
                    "and as mar_cache_attn_fwd_scores (the attention also sums the generating "
                    "queries' probabilities per head) then mar_refresh_select; per layer-2 call",
            "separate_us": avg_us["layer2_separate"], "fused_us": avg_us["layer2_fused"],
            "saved_us": avg_us["layer2_separate"] - avg_us["layer2_fused"]},
        "locality": loc,
        "c5_decode": c5,
        "attn_median_us": attn_median_us,
        "attn_frac_of_copy": (achieved / copy_gbs) if copy_gbs else None,
        "fused_frac_of_copy": (achieved_fused / copy_gbs) if copy_gbs else None,
        "attn_bytes_per_call": bytes_call,
        "attn_tok_per_s": cfg.B * cfg.A / (avg_us["attn"] * 1e-6),
        "copy_gbs": copy_gbs,
        "wall_s_timed": wall,
        "host_issue_ms_per_step": issue * 1e3 / args.steps,
    })
    print(json.dumps(line))


if __name__ == "__main__":
    main()
