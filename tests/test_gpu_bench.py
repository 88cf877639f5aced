"""bench.py end to end on the GPU at a short setting: one JSON line on stdout
with the fields the benchmark contract names, a roofline object for the
attention kernel and an oracle baseline."""
import json
import os
import subprocess
import sys

import pytest

from helpers import note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    note(f"bench.py {' '.join(args)}")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def _check_contract(d, steps, warmup):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["data"] == "synthetic" and "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and 0 < r["frac"] < 1
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)


def test_bench_lvsa_line():
    d = _bench("--workload", "wan1.3b-1x", "--steps", "2", "--warmup", "1", "--no-dense", "--cpu-seconds", "1")
    _check_contract(d, 2, 1)
    assert d["dtype"] == "bf16" and d["config"]["workload"] == "wan2.1-1.3b-1x-lvsa-full"
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]


def test_bench_draft_line():
    d = _bench("--workload", "hunyuan-draft", "--steps", "2", "--warmup", "1", "--dense-steps", "1", "--cpu-seconds",
               "1")
    _check_contract(d, 2, 1)
    assert set(d["stage_ms"]) == {"mask", "attn", "scatter"}
    assert d["speedup_vs_dense"] > 1 and d["cpu_baseline"]["kind"] == "oracle"
    assert d["config"]["flop_block_area_per_call"] >= d["config"]["flop_per_call"]
