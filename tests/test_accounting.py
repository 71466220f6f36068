"""Bytes-per-parameter accounting of the two state layouts, pinned to the
memory figures the pages print (tests/golden/pages_memory_accounting.json)."""
import json
import os

import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MiB = 1 << 20


@pytest.fixture(scope="module")
def acc():
    return json.load(open(os.path.join(GOLDEN, "pages_memory_accounting.json")))


def test_resident_bytes_match_breakdown(acc):
    mixed = acc["bf16_mixed_breakdown"]
    pure = acc["bf16_pure_breakdown"]
    per_mixed = mixed["optim"] + mixed["grad"] + sum(mixed["weights"])
    per_pure = sum(pure["optim"]) + pure["grad"] + pure["weights"]
    assert per_mixed == sum(workloads.RESIDENT_BYTES["mixed"].values()) == 16
    assert per_pure == sum(workloads.RESIDENT_BYTES["kahan"].values()) == 10
    # optimizer-state share of each layout: fp32 m+v = 8; bf16 m+v + bf16 comp = 4+2
    r = workloads.RESIDENT_BYTES
    assert r["mixed"]["m"] + r["mixed"]["v"] == mixed["optim"]
    assert [r["kahan"]["m"] + r["kahan"]["v"], r["kahan"]["c"]] == pure["optim"]
    assert [r["mixed"]["master"], r["mixed"]["p"]] == mixed["weights"]
    assert round(mixed["n_params_billion"] * per_mixed, 1) == mixed["total_gb"]
    assert round(pure["n_params_billion"] * per_pure, 1) == pure["total_gb"]
    assert round(mixed["total_gb"] - pure["total_gb"], 1) == acc["theoretical_diff_gb"]["value"]


def test_measured_train_delta_is_16_and_10_bytes_per_param(acc):
    """The train-phase allocation deltas of the two measured runs, with the real
    OPT-1.3B count (the workload list plus the final LayerNorm, 2 x 2048) and MB
    read as MiB, come to 16.0 and 10.0 bytes per parameter -- the totals of the
    two theoretical breakdowns -- and the init delta to 4.0 (fp32 weights)."""
    n_real = workloads.get("opt_1_3b").total + 2 * 2048
    mixed = acc["measured_mixed_mb"]["train_mem_gpu_alloc_delta"] * MiB / n_real
    pure = acc["measured_pure_mb"]["train_mem_gpu_alloc_delta"] * MiB / n_real
    init = acc["measured_mixed_mb"]["init_mem_gpu_alloc_delta"] * MiB / n_real
    assert abs(mixed - 16.0) < 0.01 and abs(pure - 10.0) < 0.01 and abs(init - 4.0) < 0.01
    assert abs((mixed - pure) - 6.0) < 0.01


def test_zero_expected_saving(acc):
    z = acc["zero_expected_saving"]
    per = z["fp32_optim_states"] * 4 + z["master_16bit"] * 2
    saving_mb = z["n_params_million"] * per * (1 - 1 / z["data_parallel_size"])
    assert round(saving_mb) == z["expected_mb"]
    # a rank's ZeRO shard of the BERT list holds a quarter of the state
    wl = workloads.get("bert_52m")
    b, e = wl.shard(0)
    assert e - b == wl.total // 4 == 13_059_840


def test_step_traffic_per_param():
    assert workloads.traffic_per_param("mixed") == 28
    assert workloads.traffic_per_param("kahan") == 18
    assert workloads.traffic_per_param("mixed") + workloads.traffic_per_param("check_f16") == 30


def test_bench_refuses_more_than_one_gpu():
    """bench.py times one GPU's share; asked for more it exits with a message and
    touches no GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
