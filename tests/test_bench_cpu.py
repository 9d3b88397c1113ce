"""Host-side pieces of the benchmark and the entry points (no GPU)."""
import os
import subprocess
import sys

import numpy as np

import bench
from workloads import CONFIGS, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_of_the_tiny_config():
    d = make_inputs(CONFIGS[1])
    w = bench.algorithmic_work(d)
    # 264 cached tokens of 1152 B, 16 query rows of q (1152 B), out (1024 B), lse (4 B)
    assert w["kv_bytes"] == 264 * 1152
    assert w["bytes"] == 264 * 1152 + 16 * (1152 + 1024 + 4)
    # 2 (576 + 512) flop per (row, visible key): 8 heads x 264 keys
    assert w["flops"] == 2 * (576 + 512) * 8 * 264


def test_algorithmic_work_counts_only_visible_keys_under_causal_masking():
    cfg = CONFIGS[3].with_(batch=2, seqlen_rule="fixed", seqlens_fixed=(1, 10), h_q=4)
    d = make_inputs(cfg, seed=1)
    w = bench.algorithmic_work(d)
    # token 0 sees L-1 keys, token 1 sees L keys: (0 + 1) + (9 + 10) = 20 pairs per head
    assert w["flops"] == 2 * (576 + 512) * 4 * 20


def test_cpu_baseline_reports_the_oracle_rate():
    d = make_inputs(CONFIGS[1])
    r = bench.cpu_baseline(d, budget_s=0.2)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert r["cores"] >= 1


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_entry_points_exist():
    import __graft_entry__ as g
    assert callable(g.build) and callable(g.smoke)
