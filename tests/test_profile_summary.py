"""CPU tests of the rocprofv3 summaries behind profiles/ (no GPU needed).

The committed SQ, traffic and trace summaries are computed by
latent_kv_cache_chunk_amd.profile_summary; these tests feed it small
hand-made rocprofv3 CSV files whose answers follow from the definitions:
bytes scaled by the calibration copy, the clock as GRBM_GUI_ACTIVE per XCD over
the dispatch's own duration, matrix-core busy as MFMA busy cycles over all
SIMD cycles, and the first (warmup) dispatch of a counter run left out.
"""

import csv
import json
import re
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
ATT = ("void mla::attend_bf16_kernel<192>(unsigned short const*, long, int, unsigned short const*, int, int, "
       "float*, float*, int, long, int, float, mla::Visibility, long const*, long, mla::PartitionHeader*)")
OTHER = "void mla::upproj_bf16_kernel<192, false>(float const*)"
COPY = "void at::native::vectorized_elementwise_kernel<8, neg>(int)"


def _run(*args):
    r = subprocess.run([sys.executable, "-m", "latent_kv_cache_chunk_amd.profile_summary", *map(str, args)],
                       cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return r.stdout


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d, k, c, v, t0, t1 in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v,
                        "Start_Timestamp": t0, "End_Timestamp": t1})


def test_sq_drops_warmup_and_derives_clock_and_busy(tmp_path):
    rows = []
    # warmup dispatch: inflated GRBM (it would imply 3 GHz), must be ignored
    rows += [(1, ATT, "GRBM_GUI_ACTIVE", 8 * 3.0e6, 0, 1_000_000),
             (1, ATT, "SQ_VALU_MFMA_BUSY_CYCLES", 1.0e9, 0, 1_000_000)]
    # two timed dispatches of 1 ms each at 1.8 and 1.6 GHz, MFMA busy 1.2e9 cycles
    for d, ghz in ((2, 1.8), (3, 1.6)):
        cyc = ghz * 1e9 * 1e-3
        rows += [(d, ATT, "GRBM_GUI_ACTIVE", 8 * cyc, 10_000_000 * d, 10_000_000 * d + 1_000_000),
                 (d, ATT, "SQ_VALU_MFMA_BUSY_CYCLES", 1.2e9, 10_000_000 * d, 10_000_000 * d + 1_000_000)]
    rows += [(4, OTHER, "GRBM_GUI_ACTIVE", 1.0, 0, 10), (4, OTHER, "SQ_VALU_MFMA_BUSY_CYCLES", 1.0, 0, 10)]
    p = tmp_path / "sq.csv"
    _counters(p, rows)
    out = tmp_path / "sq.md"
    text = _run("sq", p, "--workload", "wan480p", "--duration-us", "1000", "--command", "cmd", "--out", out)
    assert "Means over 2 attention dispatches" in text
    assert "**1.60-1.80 GHz**" in text
    # busy = 1.2e9 / (1024 * cycles per XCD): 1.2e9 / (1024 * 1.8e6) = 65.1%, / (1024 * 1.6e6) = 73.2%
    assert "**65.1-73.2%**" in text
    assert "| GRBM_GUI_ACTIVE | 1.36e+07 |" in text     # mean of 8*1.8e6 and 8*1.6e6


def test_sq_refuses_a_run_without_the_kernel(tmp_path):
    p = tmp_path / "sq.csv"
    _counters(p, [(1, OTHER, "GRBM_GUI_ACTIVE", 1.0, 0, 10)])
    r = subprocess.run([sys.executable, "-m", "latent_kv_cache_chunk_amd.profile_summary", "sq", str(p),
                        "--workload", "wan480p", "--duration-us", "1", "--command", "c",
                        "--out", str(tmp_path / "o.md")], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    # the copy reads 1 GiB but FETCH_SIZE reports half (KiB): scale 2; WRITE_SIZE reports all: scale 1
    gib_kib = (1 << 30) / 1024
    fetch = [(1, COPY, "FETCH_SIZE", gib_kib / 2, 0, 1), (2, ATT, "FETCH_SIZE", 1000.0, 0, 1),
             (3, ATT, "FETCH_SIZE", 3000.0, 0, 1)]
    write = [(1, COPY, "WRITE_SIZE", gib_kib, 0, 1), (2, ATT, "WRITE_SIZE", 500.0, 0, 1),
             (3, ATT, "WRITE_SIZE", 500.0, 0, 1)]
    pf, pw = tmp_path / "f.csv", tmp_path / "w.csv"
    _counters(pf, fetch)
    _counters(pw, write)
    js, md = tmp_path / "t.json", tmp_path / "t.md"
    _run("traffic", pf, pw, "--workload", "wan480p", "--command-fetch", "cf", "--command-write", "cw",
         "--out-json", js, "--out-md", md)
    t = json.loads(js.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0)
    assert t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == round(2000.0 * 1024 * 2.0)     # mean 2000 KiB, scaled x2
    assert t["write_bytes_per_launch"] == round(500.0 * 1024)
    sys.path.insert(0, str(ROOT))
    import bench
    assert t["kernel_source_hash"] == bench.kernel_source_hash(192)


def test_bench_ignores_traffic_of_another_kernel_source(tmp_path, monkeypatch):
    sys.path.insert(0, str(ROOT))
    import bench
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda d_c=192: "abc")
    path = prof / "attend_traffic_wan480p.json"
    path.write_text(json.dumps({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic("wan480p", 192) is None        # counted on other kernel sources
    path.write_text(json.dumps({"kernel_source_hash": "abc", "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic("wan480p", 192) == 123
    assert bench.load_traffic("wan480p_b8", 192) is None     # no profile for that workload


def test_trace_summary_means_exclude_warmup(tmp_path):
    stats = tmp_path / "s.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage",
                                          "MinNs", "MaxNs", "StdDev"])
        w.writeheader()
        w.writerow({"Name": ATT, "Calls": 4, "TotalDurationNs": 0, "AverageNs": 2500.0, "Percentage": 100,
                    "MinNs": 1000, "MaxNs": 5500, "StdDev": 0})
    trace = tmp_path / "t.csv"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d in (5500, 1000, 2000, 3000):          # the first (warmup) is the slow one
            w.writerow({"Kernel_Name": ATT, "Start_Timestamp": 0, "End_Timestamp": d})
    out = tmp_path / "o.md"
    text = _run("trace", stats, "--title", "T", "--command", "C", "--kernel-trace", trace, "--skip", "1",
                "--out", out)
    row = [l for l in text.splitlines() if l.startswith("| attend_bf16_kernel<192> | 3 |")]
    assert row and re.search(r"\| 2\.0 \| 2\.0 \|$", row[0]), text
