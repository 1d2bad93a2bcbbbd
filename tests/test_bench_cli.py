"""Host-side checks of bench.py (no GPU): the single-GPU guard, the algorithmic
byte count of the attention roofline, and the rule that the counter-measured
traffic is reported only for the kernel source it was taken on."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_attention_algorithmic_bytes():
    b = load_bench()
    # MAR-L layer: 128 sequences x 16 heads, A = 48 active, Nc = 272 cached, D = 64, bf16.
    # Q_A, K_A, V_A read and out written (4 x 48 rows), 272 cached K and V rows read,
    # the 272-entry int32 list read once per sequence.
    per_unit = (4 * 48 + 2 * 272) * 64 * 2
    assert b.attn_bytes(128, 16, 48, 272, 64) == 128 * 16 * per_unit + 128 * 272 * 4
    assert b.attn_bytes(128, 16, 48, 272, 64) == 193077248
    # fp32 doubles the row bytes, not the list
    assert b.attn_bytes(1, 1, 8, 56, 64, elem=4) == (4 * 8 + 2 * 56) * 64 * 4 + 56 * 4
    # the fused call also writes the 48 fresh K and V rows into the caches
    assert b.fused_bytes(128, 16, 48, 272, 64) == 193077248 + 2 * 128 * 16 * 48 * 64 * 2
    assert b.fused_bytes(128, 16, 48, 272, 64) == 218243072


def test_ragged_update_algorithmic_bytes():
    b = load_bench()
    # one sequence, one head, 10 tokens, 3 recomputed: 4 x 3 fresh rows (Q, K,
    # V read, out written), 2 x 7 reused rows read, 2 x 3 rows written into
    # the caches, the 10-entry list
    assert b.ragged_update_bytes(1, 10, 64, [3]) == (12 + 14 + 6) * 128 + 40
    # per sequence, summed: counts 0 and 10 (nothing and everything recomputed)
    assert b.ragged_update_bytes(2, 10, 64, [0, 10]) == 2 * (20 + 60) * 128 + 2 * 40


def test_traffic_only_for_the_measured_source(tmp_path):
    b = load_bench()
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"kernel_source_sha256_16": b.source_hash(str(src)),
                               "kernels": {"fused": {"hbm_bytes_per_launch": 123.0},
                                           "attention": {"hbm_bytes_per_launch": 45.0}}}))
    b.TRAFFIC_FILE, b.ATTN_SRC = str(rec), str(src)
    assert b.load_traffic("fused") == 123.0 and b.load_traffic("attention") == 45.0
    assert b.load_traffic("other") is None
    src.write_text("// kernel v2\n")  # the source changed since the counters were taken
    assert b.load_traffic("fused") is None
    rec.write_text("not json")
    assert b.load_traffic("fused") is None
    os.remove(rec)
    assert b.load_traffic("fused") is None



def test_headline_record_contract():
    """The fields the one-line record must carry, their types, and the value
    and roofline arithmetic, at the MAR-L step shape with made-up timings."""
    b = load_bench()
    from mar_workloads import CONFIGS
    cfg = CONFIGS["mar_l"]
    cpu = {"value": 1.0, "unit": "tok/s", "cores": 16, "kind": "oracle", "sample": "s"}
    rec = b.headline_record(cfg, 30, 100, 10, 1.5, 5400.0, 1.9e8, cpu)
    required = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"}
    assert required <= set(rec)
    assert rec["n_gpus"] == 1 and rec["steps"] == 100 and rec["warmup"] == 10
    assert rec["higher_is_better"] is True and rec["scaling"] == "weak"
    assert rec["vs_baseline"] is None and rec["dtype"] == "bf16" and rec["unit"] == "tok/s"
    # 128 sequences x 48 active queries x 30 layers per 1.5 ms step
    assert rec["value"] == 128 * 48 * 30 / 1.5e-3
    assert rec["config"]["workload"] == "mar_l_decode_step" and "model" not in rec["config"]
    r = rec["roofline"]
    assert set(r) == {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["frac"] == 5400.0 / 8000.0 and r["traffic"] == 1.9e8
    assert rec["cpu_baseline"] is cpu
    json.dumps(rec)  # serialisable as one line


def test_full_attention_roofline_bound():
    """The full-attention layer's roofline is chosen by its intensity against the
    bf16 ridge (2500 TFLOP/s over 8 TB/s = 312.5 flop/B): MAR-L's 320-token layer
    (4 B H N^2 D flops over 4 B H N D bf16 bytes = N/2 = 160 flop/B) is HBM-bound,
    the high-res 1088-token layer (544 flop/B) matrix-core-bound."""
    b = load_bench()
    assert b.RIDGE_FLOP_PER_BYTE == 312.5
    B, H, N, D = 128, 16, 320, 64
    flops, nbytes = 4 * B * H * N * N * D, 4 * B * H * N * D * 2
    r = b.roofline_for(flops, nbytes, 77.0e-6)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["flop_per_byte"] == 160.0
    assert abs(r["achieved"] - nbytes / 77.0e-6 / 1e9) < 1e-6 and r["frac"] == r["achieved"] / 8000.0
    B, N = 64, 1088
    flops, nbytes = 4 * B * H * N * N * D, 4 * B * H * N * D * 2
    r = b.roofline_for(flops, nbytes, 356.0e-6)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["flop_per_byte"] == 544.0
    assert r["frac"] == r["achieved"] / 2500.0
