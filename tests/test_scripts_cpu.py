"""Static checks of the repository's scripts on the CPU: every name a function of bench.py or
__graft_entry__.py reads as a global exists at module level or in builtins (a misspelt or
out-of-scope name would only fail where a GPU runs it), and bench.py refuses more than one GPU."""

import builtins
import os
import subprocess
import symtable
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def unresolved_globals(path):
    src = open(path, encoding="utf-8").read()
    top = symtable.symtable(src, path, "exec")
    module_names = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    missing = []

    def walk(tab):
        for child in tab.get_children():
            for sym in child.get_symbols():
                if sym.is_global() and sym.is_referenced():
                    n = sym.get_name()
                    if n not in module_names and not hasattr(builtins, n):
                        missing.append((child.get_name(), n))
            walk(child)

    walk(top)
    return missing


@pytest.mark.parametrize("script", ["bench.py", "__graft_entry__.py"])
def test_no_unresolved_global_names(script):
    assert unresolved_globals(os.path.join(ROOT, script)) == []


def test_bench_refuses_several_gpus():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_cpu_baseline_record():
    """The oracle's timing record: its fields, a positive rate, and a sample description that
    counts the whole passes over the row when one pass is shorter than the budget."""
    sys.path.insert(0, ROOT)
    import bench
    from transformer_causal_attention_amd.workloads import Workload

    w = Workload("tiny", 1, 96, 4, 2, 64, "bf16", 1.0, 10000.0, True, 1)
    r = bench.cpu_baseline(w, budget_s=0.4, rows_per_task=32)
    assert set(r) == {"value", "unit", "cores", "kind", "sample", "seconds", "host_cores", "blas_threads_per_worker",
                      "workers"}
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] >= 1
    # one worker process per core of the affinity mask (at most one per task), one BLAS thread each
    assert r["cores"] == r["workers"] == min(len(os.sched_getaffinity(0)), 4 * 3) and r["blas_threads_per_worker"] == 1
    assert r["host_cores"] == len(os.sched_getaffinity(0))
    assert r["value"] > 0 and r["seconds"] >= 0.4
    assert "whole passes" in r["sample"] and "tiny" in r["sample"]


def test_bench_counts():
    """The benchmark's algorithmic counts: 2 B Hq S^2 d FLOPs for a causal call (4 B Hq S^2 d
    without the mask), 4 d FLOPs per visible (row, key) pair for sampled rows (counted by brute
    force here), and q, k, v, out in bf16 plus an fp32 lse for the bytes."""
    sys.path.insert(0, ROOT)
    import bench
    from transformer_causal_attention_amd.workloads import WORKLOADS, Workload

    w = WORKLOADS["llama3_8b"]
    assert bench.flops(w) == 2 * 1 * 32 * 2048 * 2048 * 128
    assert bench.algorithmic_bytes(w) == (2 * 2048 * 32 * 128 + 2 * 2048 * 8 * 128) * 2 + 4 * 32 * 2048
    t = Workload("t", 2, 37, 6, 3, 64, "bf16", 1.0, 10000.0, True, 1)
    rows = [0, 5, 36]
    pairs = sum(1 for i in rows for j in range(t.S) if j <= i)
    assert bench.flops(t, rows) == 4 * t.d * pairs * t.B * t.Hq
    tf = Workload("t", 2, 37, 6, 3, 64, "bf16", 1.0, 10000.0, False, 1)
    assert bench.flops(tf) == 4 * 2 * 6 * 37 * 37 * 64
    assert bench.flops(tf, rows) == 4 * tf.d * len(rows) * tf.S * tf.B * tf.Hq
