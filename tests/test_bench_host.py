"""Host logic of bench.py (no GPU): the committed-profile readers, the counter and trace
summaries built from rocprofv3 CSV files, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_kernel_source_sha_is_stable():
    a, b = bench.kernel_source_sha(), bench.kernel_source_sha()
    assert a == b and len(a) == 64 and int(a, 16) >= 0


def test_profile_fields_reads_key_value_lines(tmp_path):
    p = tmp_path / "p.md"
    p.write_text("# title\n\n- kernel: `k<1>`\n- kernel_duration_mean_us: 4.5\nnot a field: x\n- bad line\n")
    assert bench._profile_fields(str(p)) == {"kernel": "k<1>", "kernel_duration_mean_us": "4.5"}
    assert bench._profile_fields(str(tmp_path / "missing.md")) == {}


def test_committed_readers_void_on_source_change(tmp_path, monkeypatch):
    """The traffic and trace figures are read only while the kernel sources hash to the recorded
    sha256; a summary recorded for other sources gives None."""
    sha = bench.kernel_source_sha()
    good = tmp_path / "trace.md"
    good.write_text(f"- kernel: `k`\n- source_sha256: `{sha}`\n- kernel_duration_mean_us: 5.0\n"
                    "- kernel_duration_median_us: 4.9\n")
    stale = tmp_path / "stale.md"
    stale.write_text("- kernel: `k`\n- source_sha256: `00`\n- kernel_duration_mean_us: 5.0\n")
    monkeypatch.setattr(bench, "TRACE_PROFILE", str(good))
    kt = bench.committed_kernel_trace(10_000_000)
    assert kt["kernel_duration_mean_us"] == 5.0
    assert kt["achieved"] == pytest.approx(2000.0) and kt["frac"] == pytest.approx(2000.0 / bench.HBM_PEAK_GBS, abs=1e-4)
    monkeypatch.setattr(bench, "TRACE_PROFILE", str(stale))
    assert bench.committed_kernel_trace(10_000_000) is None
    traffic = tmp_path / "traffic.md"
    traffic.write_text(f"- source_sha256: `{sha}`\n- hbm_bytes_per_launch: 11548043\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(traffic))
    assert bench.committed_traffic() == 11548043
    traffic.write_text("- source_sha256: `ff`\n- hbm_bytes_per_launch: 11548043\n")
    assert bench.committed_traffic() is None


def _counter_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "1_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_pmc_summary_scales_by_the_copy(tmp_path):
    """FETCH_SIZE of the copy reads half its bytes, WRITE_SIZE all of them: the GEMV's counters
    are scaled by the same factors, and the summary states the ratio to the algorithmic bytes."""
    kib = 1024.0
    copy_bytes = 256 << 20
    g = "void bitlinear::k_gemv<1, 1, 6, true, 8, true>(bitlinear::GemvArgs)"
    _counter_csv(tmp_path / "gf", [(g, "FETCH_SIZE", 5000.0)] * 3)
    _counter_csv(tmp_path / "gw", [(g, "WRITE_SIZE", 40.0)] * 3)
    _counter_csv(tmp_path / "cf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", copy_bytes / kib / 2)])
    _counter_csv(tmp_path / "cw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", copy_bytes / kib)])
    text = bench.pmc_summary(str(tmp_path / "gf"), str(tmp_path / "gw"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                             ["cmd one", "cmd two"])
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k] = v.strip("`")
    assert fields["fetch_factor"] == "2.0000" and fields["write_factor"] == "1.0000"
    assert int(fields["hbm_bytes_per_launch"]) == int(5000.0 * kib * 2 + 40.0 * kib)
    k, n = bench.DECODE_SHAPES[1]
    assert int(fields["algorithmic_bytes_per_launch"]) == n * k // 4 + 4 * k + 4 + 4 * n
    assert fields["source_sha256"] == bench.kernel_source_sha()
    assert "cmd one" in text and "cmd two" in text


def test_trace_summary_takes_the_timed_replays(tmp_path, capsys):
    """The roofline kernel's launches in the trace are, in order, 3 warm-up calls, one untimed
    replay and `trials` timed replays of L launches, then 50 single calls; the summary measures
    the timed replays only."""
    L, trials = 4, 2
    name = "void bitlinear::k_gemv<1, 1, 6, true, 8, true>(bitlinear::GemvArgs)"
    rows, t = [], 0
    n_launch = 3 + L * (1 + trials) + 50
    for i in range(n_launch):
        timed = 3 + L <= i < 3 + L * (1 + trials)
        dur = 5000 if timed else 9000
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
        t += dur + 1000
    rows.append({"Kernel_Name": "other", "Start_Timestamp": 0, "End_Timestamp": 1})
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "x_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    plain = tmp_path / "plain.json"
    plain.write_text(json.dumps({"us_per_launch": 4.7, "achieved": 2400.0}) + "\n")
    traced = tmp_path / "traced.json"
    traced.write_text(json.dumps({"us_per_launch": 6.0, "graph_launches": L, "graph_trials": trials}) + "\n")
    bench.trace_summary(str(d), str(plain), str(traced), "a; b")
    out = capsys.readouterr().out
    fields = dict(line[2:].split(": ", 1) for line in out.splitlines() if line.startswith("- ") and ": " in line)
    assert fields["launches_timed"].startswith(f"{L * trials} ")
    assert float(fields["kernel_duration_mean_us"]) == pytest.approx(5.0)
    assert float(fields["traced_launch_to_launch_us"]) == pytest.approx((L * trials * 6000 - 1000) / (L * trials) / 1e3)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
