"""Summaries of rocprofv3 output for the committed profiles.

    python -m latent_kv_cache_chunk_amd.profile_summary trace <run_kernel_stats.csv> --title T --command C --out F.md
    python -m latent_kv_cache_chunk_amd.profile_summary traffic <fetch_counter_collection.csv>
        <write_counter_collection.csv> --workload wan480p --command-fetch C1 --command-write C2
        --out-json profiles/attend_traffic_wan480p.json --out-md F.md

    python -m latent_kv_cache_chunk_amd.profile_summary sq <pass1_counter_collection.csv> [<pass2...>]
        --workload wan480p --duration-us D --command C1 [--command C2] --out F.md

`trace` turns the kernel statistics table into markdown.  `sq` averages the
SQ/GRBM counters of the attention kernel over its dispatches (warmup dropped)
and derives the matrix-core busy fraction and the shader clock per dispatch.  `traffic` converts
FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernel into bytes,
scaled by what the same counters read for the probe's calibration kernel (an
elementwise negation that reads and writes a known number of bytes once),
and records the attention source hash so a later kernel change invalidates it.
"""

from __future__ import annotations

import argparse
import csv
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def short_name(name: str) -> str:
    m = re.search(r"mla::(?:\w+::)*(\w+(?:<[^>]*>)?)\(", name)
    if m:
        return m.group(1)
    return name.split("(")[0][-80:]


def cmd_trace(a) -> None:
    rows = list(csv.DictReader(open(a.stats)))
    lines = [f"# {a.title}", "", "Command (repo root, one MI355X):", "", f"    {a.command}", ""]
    if a.note:
        lines += [a.note, ""]
    lines += ["| Kernel | Calls | Avg (us) | Min (us) | Max (us) | Share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    if a.kernel_trace:
        # mean over the timed steps only: drop each kernel's first `skip` dispatches (warmup)
        per = defaultdict(list)
        for r in csv.DictReader(open(a.kernel_trace)):
            per[short_name(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        lines += ["", f"Excluding the first {a.skip} dispatches of each kernel (warmup):", "",
                  "| Kernel | Dispatches | Avg (us) | Median (us) |", "|---|---|---|---|"]
        for k, v in per.items():
            v = sorted(v[a.skip:]) if len(v) > a.skip else sorted(v)
            t = [x / 1e3 for x in v]
            lines.append(f"| {k} | {len(t)} | {sum(t) / len(t):.1f} | {t[len(t) // 2]:.1f} |")
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(path: str, counter: str):
    """Per-kernel list of per-dispatch counter values."""
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def _pick(per, pattern: str):
    hits = [(k, v) for k, v in per.items() if re.search(pattern, k)]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {pattern!r}, found {[k[:60] for k, _ in hits]}")
    return hits[0]


# MI355X: 256 compute units in 8 XCDs, 4 SIMDs (one matrix core each) per CU.
CUS, XCDS, SIMDS_PER_CU = 256, 8, 4


def cmd_sq(a) -> None:
    """SQ/GRBM counters of the attention kernel, per dispatch.  The first
    `skip` dispatches of a pass are dropped: the first one's GRBM_GUI_ACTIVE
    also counts cycles outside the kernel (it implies more than the part's
    2.4 GHz).  The clock of a dispatch is its GRBM_GUI_ACTIVE per XCD over its
    own duration in the same run (the counter runs are slower than unprofiled
    ones; the ratio is what the counters measure)."""
    sys.path.insert(0, ROOT)
    import bench
    from latent_kv_cache_chunk_amd import synth
    d_c = synth.WORKLOADS[a.workload].d_c
    pattern = r"mla::(wide::)?" + bench.attend_kernel(d_c)
    name, means, clocks, busys, durs, n_kept = None, {}, [], [], [], 0
    for path in a.passes:
        disp = defaultdict(dict)
        for r in csv.DictReader(open(path)):
            if not re.search(pattern, r["Kernel_Name"]):
                continue
            name = r["Kernel_Name"]
            d = disp[int(r["Dispatch_Id"])]
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["_dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        kept = [disp[k] for k in sorted(disp)][a.skip:]
        if not kept:
            raise SystemExit(f"no dispatch of {pattern!r} left in {path}")
        n_kept = len(kept)
        for c in kept[0]:
            if c != "_dur_us":
                means[c] = sum(d[c] for d in kept) / len(kept)
        for d in kept:
            if "GRBM_GUI_ACTIVE" in d:
                cyc = d["GRBM_GUI_ACTIVE"] / XCDS
                clocks.append(cyc / d["_dur_us"] / 1e3)
                durs.append(d["_dur_us"])
                if "SQ_VALU_MFMA_BUSY_CYCLES" in d:
                    busys.append(d["SQ_VALU_MFMA_BUSY_CYCLES"] / (CUS * SIMDS_PER_CU * cyc))
    lines = [f"# SQ counters: {short_name(name)}, workload {a.workload}", "",
             "Commands (repo root, one MI355X; one counter set per pass):", ""]
    lines += [f"    {c}" for c in a.command]
    lines += ["", f"Means over {n_kept} attention dispatches of a pass (the first {a.skip} dropped: warmup). "
              f"Unprofiled, the kernel takes {a.duration_us:.1f} us (kernel trace of the same sources); under "
              "the counters its dispatches ran " + (f"{min(durs):.1f}-{max(durs):.1f} us." if durs else "-"), "",
              "| Counter | Value per dispatch |", "|---|---|"]
    lines += [f"| {k} | {v:.4g} |" for k, v in sorted(means.items())]
    rng = lambda v, f: f(v[0]) if f(min(v)) == f(max(v)) else f"{f(min(v))}-{f(max(v))}"
    derived = []
    if clocks:
        derived.append(f"* Shader clock: GRBM_GUI_ACTIVE / {XCDS} XCDs over each dispatch's duration = "
                       f"**{rng(clocks, lambda x: f'{x:.2f}')} GHz**.")
    if busys:
        derived.append(f"* Matrix cores busy: SQ_VALU_MFMA_BUSY_CYCLES / ({CUS * SIMDS_PER_CU} SIMDs x "
                       f"GRBM_GUI_ACTIVE / {XCDS}) = **{rng(busys, lambda x: f'{100 * x:.1f}')}%** of the launch.")
    if "SQ_WAVE_CYCLES" in means and "SQ_WAIT_INST_ANY" in means:
        derived.append(f"* Waves waiting on a dependency: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES = "
                       f"{100 * means['SQ_WAIT_INST_ANY'] / means['SQ_WAVE_CYCLES']:.1f}%.")
    if "SQ_INSTS_LDS" in means and "SQ_LDS_BANK_CONFLICT" in means:
        derived.append(f"* LDS bank-conflict cycles per LDS instruction: "
                       f"{means['SQ_LDS_BANK_CONFLICT'] / means['SQ_INSTS_LDS']:.2f}.")
    if derived:
        lines += ["", "Derived:", ""] + derived
    if a.note:
        lines += ["", a.note]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_traffic(a) -> None:
    sys.path.insert(0, ROOT)
    import bench
    from latent_kv_cache_chunk_amd import synth
    d_c = synth.WORKLOADS[a.workload].d_c
    fetch = _counter(a.fetch, "FETCH_SIZE")
    write = _counter(a.write, "WRITE_SIZE")
    _, f_copy = _pick(fetch, r"neg")
    _, w_copy = _pick(write, r"neg")
    pattern = r"mla::(wide::)?" + bench.attend_kernel(d_c)
    name, f_att = _pick(fetch, pattern)
    _, w_att = _pick(write, pattern)
    kib = 1024.0
    copy_bytes = float(a.copy_bytes)
    f_scale = copy_bytes / (sum(f_copy) / len(f_copy) * kib)
    w_scale = copy_bytes / (sum(w_copy) / len(w_copy) * kib)
    f_b = sum(f_att) / len(f_att) * kib * f_scale
    w_b = sum(w_att) / len(w_att) * kib * w_scale
    out = {
        "kernel": short_name(name), "workload": a.workload,
        "kernel_source_hash": bench.kernel_source_hash(d_c),
        "hbm_bytes_per_launch": round(f_b + w_b),
        "fetch_bytes_per_launch": round(f_b), "write_bytes_per_launch": round(w_b),
        "fetch_scale": f_scale, "write_scale": w_scale,
        "calibration": f"elementwise negation of {int(copy_bytes)} bytes (reads and writes each once)",
        "dispatches": {"attend": len(f_att), "copy": len(f_copy)},
        "commands": {"fetch": a.command_fetch, "write": a.command_write},
    }
    json.dump(out, open(a.out_json, "w"), indent=1)
    md = [f"# HBM traffic: {out['kernel']}, workload {a.workload}", "",
          "Commands (repo root, one MI355X; one counter per pass):", "",
          f"    {a.command_fetch}", f"    {a.command_write}", "",
          f"Calibration: {out['calibration']}: FETCH_SIZE reads {sum(f_copy) / len(f_copy):.0f} KiB per dispatch "
          f"(scale {f_scale:.4f}), WRITE_SIZE {sum(w_copy) / len(w_copy):.0f} KiB (scale {w_scale:.4f}).", "",
          "| Counter | KiB per attend dispatch (mean) | Scaled bytes |", "|---|---|---|",
          f"| FETCH_SIZE | {sum(f_att) / len(f_att):.0f} | {f_b / 1e9:.3f} GB |",
          f"| WRITE_SIZE | {sum(w_att) / len(w_att):.0f} | {w_b / 1e9:.3f} GB |", "",
          f"Total {(f_b + w_b) / 1e9:.3f} GB per launch; attention source hash {out['kernel_source_hash']}."]
    if a.note:
        md += ["", a.note]
    open(a.out_md, "w").write("\n".join(md) + "\n")
    print("\n".join(md))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--note", default="")
    t.add_argument("--kernel-trace", default="", help="run_kernel_trace.csv, for the timed-steps mean")
    t.add_argument("--skip", type=int, default=0)
    t.add_argument("--out", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("fetch")
    f.add_argument("write")
    f.add_argument("--workload", default="wan480p")
    f.add_argument("--copy-bytes", type=int, default=1 << 30)
    f.add_argument("--command-fetch", required=True)
    f.add_argument("--command-write", required=True)
    f.add_argument("--note", default="")
    f.add_argument("--out-json", required=True)
    f.add_argument("--out-md", required=True)
    q = sub.add_parser("sq")
    q.add_argument("passes", nargs="+")
    q.add_argument("--workload", default="wan480p")
    q.add_argument("--duration-us", type=float, required=True, help="unprofiled kernel time, for reference")
    q.add_argument("--skip", type=int, default=1)
    q.add_argument("--command", action="append", required=True)
    q.add_argument("--note", default="")
    q.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "traffic": cmd_traffic, "sq": cmd_sq}[a.cmd](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
