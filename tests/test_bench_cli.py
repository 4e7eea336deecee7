"""bench.py's command-line contract and the bookkeeping it reports, on the host: one GPU
only, a loud failure without a GPU, and the profile digest that decides whether stored
HBM counter figures still describe the kernels."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.skipif(torch.cuda.is_available(), reason="a GPU is present")
def test_no_gpu_fails_loudly():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")        # no result line


def test_digest_ignores_comments_and_layout_only():
    a = "int f(int x) { return x + 1; }"
    b = "// the successor\nint f(int x) {\n  return x + 1;  /* plus one */\n}\n"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_digest_covers_every_kernel_source():
    d = bench.source_digest()
    assert len(d) == 16
    csrc = os.path.join(ROOT, "hash_top_kv_amd", "csrc")
    built = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h"))}
    listed = {os.path.basename(f) for f in bench.KERNEL_SOURCES}
    assert built <= listed, built - listed


def test_counter_summary_is_used_only_for_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "cur_counters.txt").write_text("source_digest: ffffffffffffffff\n"
                                           "hbm_bytes_per_launch: 123\n")
    (prof / "old_counters.txt").write_text("source_digest: 0000000000000000\n"
                                           "hbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "ffffffffffffffff")
    assert bench.read_traffic("cur") == 123.0
    assert bench.read_traffic("old") is None
    assert bench.read_traffic("missing") is None


def test_trace_summary_separates_back_to_back_dispatches(tmp_path, monkeypatch):
    """The kernel-trace summary averages a kernel over all its dispatches and, apart, over
    those that start within 1 us of the previous dispatch's end (as launches run back to
    back without the profiler); bench.read_trace hands both to the result line."""
    import csv
    import json
    import profile_summary
    run = tmp_path / "run"
    run.mkdir()
    scan = "void hk::(anonymous namespace)::hamming_scan_kernel<4, 8, false>(unsigned int const*)"
    rows, t = [], 1_000_000
    for i in range(30):                          # isolated: 10 us gap, 13 us long
        t += 10_000
        rows.append((scan, t, t + 13_000))
        t += 13_000
    for i in range(20):                          # back to back: no gap, 12 us long
        rows.append((scan, t, t + 12_000))
        t += 12_000
    with open(run / "tr_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"])
        for n, s, e in rows:
            w.writerow([n, s, e, 256])
    with open(run / "tr_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writerow([scan, 50, 12600, 12000, 13000, 100.0])
    (tmp_path / "run.json").write_text(json.dumps({"roofline": {"alg_bytes_per_launch": 1 << 20}}))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(profile_summary, "ROOT", str(tmp_path))
    monkeypatch.setattr(profile_summary, "_digest", lambda: "ffffffffffffffff")
    args = type("A", (), {"dir": str(run), "tag": "tst", "json": str(tmp_path / "run.json"),
                          "title": "t", "cmd": "c", "out": ""})
    profile_summary.trace(args)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "ffffffffffffffff")
    tr = bench.read_trace("tst", "hamming_scan")
    assert tr["all_dispatches_avg_us"] == pytest.approx((30 * 13 + 20 * 12) / 50, abs=1e-3)
    assert tr["tight_avg_us"] == pytest.approx(12.0, abs=1e-3)
    assert tr["tight_dispatches"] == 20
    # a run of >= 20 consecutive scan dispatches: the last 20 plus the 30 before them
    assert tr["back_to_back_avg_us"] == pytest.approx((30 * 13 + 20 * 12) / 50, abs=1e-3)
