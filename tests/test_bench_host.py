"""Host-side parts of bench.py: the one-GPU guard, the summaries that turn
rocprofv3 CSV output into the committed profile records, and the kernel
code hash that ties a record to the code it was taken on."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
        "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
        "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
ATTN = "void lvsa::(anonymous namespace)::bsa_fwd_d128_kernel<1, false, 8>(lvsa::AttnArgs)"
TAIL = "void lvsa::(anonymous namespace)::bsa_fwd_d128_grp_kernel<6, true>(lvsa::AttnArgs)"
COPY = "void lvsa::(anonymous namespace)::token_permute_kernel(u32x4 const*, u32x4*, int const*, int, int, int)"


def _write(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, COLS)
        w.writeheader()
        for i, (kernel, counter, value, t0, t1) in enumerate(rows):
            r = {c: 0 for c in COLS}
            r.update(Dispatch_Id=i + 1, Kernel_Name=kernel, Counter_Name=counter, Counter_Value=value,
                     Start_Timestamp=t0, End_Timestamp=t1)
            w.writerow(r)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("extra", [["--budget", "0"], ["--workload", "hunyuan-draft", "--budget", "8"]])
def test_bad_frame_budget_is_refused(extra):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + extra, capture_output=True, text=True,
                       cwd=ROOT)
    assert r.returncode == 2 and "--budget" in r.stderr


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    mib = 64
    rows = mib * (1 << 20) // 256
    known_r, known_w = (rows * 256 + rows * 4) / 1024, rows * 256 / 1024
    # the counter reads half the copy's bytes on fetch and all of them on write
    fetch = [(COPY, "FETCH_SIZE", known_r / 2, 0, 1)] * 3 + [(ATTN, "FETCH_SIZE", 1000.0, 0, 1),
                                                             (ATTN, "FETCH_SIZE", 3000.0, 0, 1),
                                                             (TAIL, "FETCH_SIZE", 50.0, 0, 1),
                                                             (TAIL, "FETCH_SIZE", 150.0, 0, 1)]
    write = [(COPY, "WRITE_SIZE", known_w, 0, 1)] * 3 + [(ATTN, "WRITE_SIZE", 10.0, 0, 1),
                                                         (ATTN, "WRITE_SIZE", 30.0, 0, 1),
                                                         (TAIL, "WRITE_SIZE", 2.0, 0, 1),
                                                         (TAIL, "WRITE_SIZE", 4.0, 0, 1)]
    _write(tmp_path / "f", fetch)
    _write(tmp_path / "w", write)
    out = tmp_path / "t.json"
    assert bench.summarize(["traffic", "--workload", "wan1.3b-6x", "--fetch", str(tmp_path / "f"), "--write",
                            str(tmp_path / "w"), "--calib-copy-mb", str(mib), "--out", str(out)]) == 0
    t = json.loads(out.read_text())
    assert t["copy_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert t["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    # per call: the full-tile launch and the frame-tail launch
    assert t["hbm_fetch_bytes_per_launch"] == pytest.approx((2000.0 + 100.0) * 2 * 1024)
    assert t["hbm_write_bytes_per_launch"] == pytest.approx((20.0 + 3.0) * 1024)
    assert t["launches_per_call"]["bsa_fwd_d128_grp_kernel<6, true>"]["read"] == pytest.approx(100.0 * 2 * 1024)
    assert t["hbm_bytes_per_launch"] == pytest.approx(t["hbm_fetch_bytes_per_launch"] + t["hbm_write_bytes_per_launch"])
    # Q, K, V read once (bf16) and O written once (fp32)
    assert t["algorithmic_bytes_per_launch"] == 3 * 12 * 196560 * 128 * 2 + 12 * 196560 * 128 * 4
    assert t["kernel_code_sha256_16"] == bench.src_hash(*bench.LVSA_SRCS)
    assert bench.src_hash(*bench.LVSA_SRCS) != bench.src_hash(bench.ATTN_SRC)


def test_counter_summary(tmp_path):
    dur_ns = 2_000_000  # 2 ms
    gui = 8 * 2.0e9 * 2e-3  # 8 XCDs at 2 GHz for 2 ms
    a = [(ATTN, "GRBM_GUI_ACTIVE", gui, 0, dur_ns), (ATTN, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * gui / 8, 0, dur_ns),
         (ATTN, "SQ_INSTS_MFMA", 100.0, 0, dur_ns), (ATTN, "SQ_INSTS_VALU", 500.0, 0, dur_ns),
         (ATTN, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 4.0, 0, dur_ns)]
    m = [(ATTN, "GRBM_GUI_ACTIVE", gui, 0, dur_ns), (ATTN, "TCC_HIT_sum", 90.0, 0, dur_ns),
         (ATTN, "TCC_MISS_sum", 10.0, 0, dur_ns), (TAIL, "GRBM_GUI_ACTIVE", gui / 4, 0, dur_ns // 4)]
    _write(tmp_path / "a", a)
    _write(tmp_path / "m", m)
    out = tmp_path / "c.json"
    assert bench.summarize(["counters", "--workload", "wan1.3b-6x", "--passes", str(tmp_path / "a"),
                            str(tmp_path / "m"), "--out", str(out)]) == 0
    rec = json.loads(out.read_text())
    met = rec["metrics"]
    assert rec["other_launches_per_call"]["bsa_fwd_d128_grp_kernel<6, true>"]["duration_ms_under_counters"] == 0.5
    assert met["shader_clock_ghz"] == pytest.approx(2.0)
    assert met["mfma_busy_frac"] == pytest.approx(0.5)
    assert met["other_valu_per_mfma"] == pytest.approx(4.0)
    assert met["matrix_core_flop_per_launch"] == pytest.approx(4.0 * 512)
    assert met["l2_hit_rate"] == pytest.approx(0.9)
    assert met["duration_ms_under_counters"] == pytest.approx(2.0)


def test_code_hash_ignores_comments_and_whitespace(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) { return x + 1; }  // one\n")
    b.write_text("/* header */\nint  f(int x)\n{\n  return x + 1;  // two\n}\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.src_hash(str(a)) == bench.src_hash(str(b)) != bench.src_hash(str(c))


def test_records_carry_their_source(tmp_path, monkeypatch):
    """Figures taken from a committed record name the file and the code hash,
    and a record taken on other kernel code is not used."""
    src = tmp_path / "k.hip"
    src.write_text("int k() { return 1; }\n")
    (tmp_path / "profiles").mkdir()
    rec = {"kernel_code_sha256_16": bench.src_hash(str(src)), "hbm_bytes_per_launch": 123.0,
           "metrics": {"l2_hit_rate": 0.5}, "commands": ["python3 bench.py"]}
    for kind in ("traffic", "counters"):
        (tmp_path / "profiles" / f"{kind}_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    val, where = bench.traffic_for("w", str(src))
    assert val == 123.0 and where["file"] == os.path.join("profiles", "traffic_w.json")
    assert where["kernel_code_sha256_16"] == rec["kernel_code_sha256_16"] and "not this run" in where["measured"]
    ctr = bench.counters_for("w", str(src))
    assert ctr["l2_hit_rate"] == 0.5 and ctr["source"]["file"].endswith("counters_w.json")
    src.write_text("int k() { return 2; }\n")
    assert bench.traffic_for("w", str(src)) == (None, None) and bench.counters_for("w", str(src)) is None


@pytest.mark.parametrize("key", ["wan14b-6x", "wan1.3b-6x", "wan1.3b-6x-fp8", "hunyuan-draft", "hunyuan-draft-fp8"])
def test_committed_records_name_their_commands(key):
    for kind in ("traffic", "counters"):
        path = os.path.join(ROOT, "profiles", f"{kind}_{key}.json")
        if not os.path.exists(path):
            continue
        t = json.load(open(path))
        assert t["commands"] and all("bench.py" in c for c in t["commands"])
        assert len(t["kernel_code_sha256_16"]) == 16
