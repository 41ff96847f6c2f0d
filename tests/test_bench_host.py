"""Host-side logic of bench.py (CPU): which kernel family and device kernel each workload runs, and
the source digest that recorded HBM traffic is keyed to."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_tiled_attention_05_amd import workloads as W  # noqa: E402


def test_family_follows_the_forward_kernel_choice():
    # fa_api.hip: the wide-row kernel for bf16 d = 128 with N >= 4096, plain, with a causal sliding
    # window or with causal ALiBi; the 4-wave kernel for the other variants, d = 256, the other
    # causal d = 128 grids and grids past 2^16 rows; the 8-wave kernel for the rest
    assert bench.workload_family("llama3_8b_n8k_causal") == "wide"
    assert bench.workload_family("llama3_8b_gqa_n8k_causal") == "wide"
    assert bench.workload_family("long_n32k_causal") == "wide"
    assert bench.workload_family("d256_h16_n8k_causal") == "ext"
    assert bench.workload_family("outlier_b16h32_n2k") == "ext"        # N = 2048, 2^20 rows
    assert bench.workload_family("b4h16_n1k_d64") == "fwd"             # 2^16 rows, d = 64
    assert bench.workload_family("single_head_fp32") == "fwd"
    assert bench.workload_family("llama3_8b_gqa_decode_b8_n32k") == "decode"
    assert bench.workload_family("llama3_8b_n8k_causal_bwd") == "bwd"
    assert bench.workload_family("b1h16_n4k_bias") == "ext"
    assert bench.workload_family("llama3_8b_n8k_causal_alibi") == "wide"
    assert bench.device_kernel("single_head_fp32") == "fa_fwd_f32_kernel"
    assert bench.device_kernel("b4h16_n1k_d64").startswith("fa_fwd_bf16_kernel")
    assert bench.device_kernel("llama3_8b_n8k_causal").startswith("fa_fwd_wide_kernel")
    assert bench.device_kernel("outlier_b16h32_n2k").startswith("fa_fwd_ext_kernel")


def test_code_only_drops_comments_but_not_strings():
    src = 'int a; // note\n/* block\n comment */ int  b;\nconst char* s = "// kept \\" x"; char c = \'/\';'
    assert bench._code_only(src) == 'int a; int b; const char* s = "// kept \\" x"; char c = \'/\';'
    assert bench._code_only("x = 1; // a") == bench._code_only("x  =  1;   /* b */")


def test_digest_is_per_family_and_stable():
    d = {wl: bench.kernel_source_digest(wl) for wl in W.WORKLOADS}
    assert all(len(x) == 64 for x in d.values())
    assert d["llama3_8b_n8k_causal"] == d["long_n32k_causal"]           # same family, same sources
    assert d["outlier_b16h32_n2k"] == d["d256_h16_n8k_causal"]
    assert d["llama3_8b_n8k_causal"] != d["d256_h16_n8k_causal"]
    assert d["llama3_8b_n8k_causal"] != d["llama3_8b_n8k_causal_bwd"]
    assert d["llama3_8b_gqa_decode_b8_n32k"] != d["llama3_8b_n8k_causal_bwd"]
    assert bench.kernel_source_digest("llama3_8b_n8k_causal") == d["llama3_8b_n8k_causal"]


def test_recorded_traffic_entries_are_well_formed():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    for wl, r in rec.items():
        assert wl in W.WORKLOADS
        assert len(r["source_sha256"]) == 64 and r["bytes_per_launch"] > 0


def test_oracle_pool_runs_whole_batches_within_budget():
    import threading
    seen = []
    lock = threading.Lock()

    def task(i):
        def run():
            with lock:
                seen.append(i)
        return run

    # the pool goes round the tasks again until the budget is spent, in whole batches
    done, dt, workers = bench.oracle_pool([task(i) for i in range(5)], budget_s=0.3)
    assert dt >= 0.3 and done == len(seen) and done % workers == 0 and 1 <= workers <= 5
    assert set(seen) == set(range(5)) and done > 5
    assert all(seen.count(i) >= seen.count(j) for i, j in zip(range(4), range(1, 5)))
    # a zero budget still runs one full batch
    seen.clear()
    done, dt, workers = bench.oracle_pool([task(i) for i in range(50)], budget_s=0.0)
    assert done == workers == len(seen)


def test_cpu_baseline_counts_sampled_rows():
    # FLOPs of a sampled-row sample: 4 (i + 1) d per causal row i, for every head done
    w = dict(B=1, H=2, N=256, d=64, dtype="bf16", causal=(True,), seed=0, sample_rows=8)
    q, k, v = W.make_inputs(1, 2, 256, 64, "bf16", seed=0)
    r = bench.cpu_baseline(q, k, v, 0.125, True, w, 2, budget_s=0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert "sampled rows" in r["sample"] and r["cores"] >= 1


def test_parse_sclk():
    assert bench.parse_sclk("S: 94Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 94
    assert bench.parse_sclk("0: 500Mhz\n1: 2400Mhz *\n") == 2400
    assert bench.parse_sclk("0: 500Mhz\n1: 2400Mhz\n") is None
