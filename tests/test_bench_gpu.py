"""bench.py's step variants each run to the end and print one well-formed result line (GPU).

The benchmark is the measuring instrument, not the product, but its step loop schedules the
library's calls on two streams in several ways (where the gradient sort starts, two
workspaces for the next batch's sort, graph replay, forward-only shapes); each variant runs
here for a couple of steps on a small workload, in a child process as the driver runs it."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
QUICK = ["--steps", "2", "--warmup", "1", "--batches", "2", "--no-cpu-baseline", "--no-calib",
         "--no-uniform-control"]

VARIANTS = [
    ("tiny-auto", ["--workload", "tiny"]),
    ("tiny-none", ["--workload", "tiny", "--overlap-sort", "none"]),
    ("tiny-fwd", ["--workload", "tiny", "--overlap-sort", "fwd"]),
    ("tiny-bwd", ["--workload", "tiny", "--overlap-sort", "bwd"]),
    ("tiny-next", ["--workload", "tiny", "--overlap-sort", "next"]),
    ("tiny-graph", ["--workload", "tiny", "--graph"]),
    ("tiny-separate", ["--workload", "tiny", "--separate-fwd", "--overlap-sort", "none"]),
    ("tiny-hash", ["--workload", "tiny", "--hash-indices"]),
    ("small-tables-hash-next", ["--workload", "train_small_tables", "--hash-indices", "--overlap-sort", "next"]),
    ("small-tables", ["--workload", "train_small_tables"]),
    ("forward-only", ["--workload", "fwd_core"]),
]


def run_bench(args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, p.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("args", [v[1] for v in VARIANTS], ids=[v[0] for v in VARIANTS])
def test_bench_variant_prints_one_result_line(args):
    d = run_bench(args + QUICK)
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["steps"] == 2 and d["warmup"] == 1 and d["n_gpus"] == 1
    assert d["unit"] == "samples/s" and d["higher_is_better"] is True
    assert d["roofline"]["bound"] in ("hbm", "mfma", "alu")
    for c in d.get("calls", {}).values():
        assert c["ms"] >= 0
    assert d["config"]["hash_indices"] is ("--hash-indices" in args)
    for r in d.get("rooflines", [d["roofline"]]):
        assert (r["traffic"] is None) == ("traffic_gbps" not in r)
        assert r["frac"] <= 1 or "caches serve" in r.get("note", "")


def test_bench_refuses_graph_with_the_next_batch_sort():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--overlap-sort", "next", "--graph", *QUICK], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert p.returncode != 0 and "graph" in (p.stdout + p.stderr)
