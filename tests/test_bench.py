"""Host-side checks of bench.py (no GPU): the algorithmic byte counts the
roofline divides by, the one-GPU guard, and the oracle baseline's record."""
import subprocess
import sys
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_algorithmic_bytes_at_the_headline_shape():
    import bench
    b = bench.algorithmic_bytes(4096, 8, 7168)
    # S*H*2 + C*H*2 + C*4;  2*C*H*2 + C*4;  C*H*2 + 2*C*4 + S*H*2  (C = S*K)
    assert b["pack"] == 528_613_376
    assert b["group"] == 939_655_168
    assert b["combine"] == 528_744_448
    assert b["pack"] + b["group"] + b["combine"] == 1_997_012_992


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_record():
    import bench
    import oracle
    import synth
    d = synth.make_plan_inputs("small", all_ranks_x=False)
    ref = oracle.plan(d["topk_ids"], d["R"], d["E"], d["S"], d["K"], 0)
    rec = bench.cpu_baseline(d, ref, budget_s=0.0)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["unit"] == "GB/s"
    assert rec["value"] > 0 and rec["routes_per_s_plan"] > 0
    assert "passes" in rec["sample"]
