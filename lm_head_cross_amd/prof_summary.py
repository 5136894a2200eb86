"""Summaries of rocprofv3 output for `profiles/`, and the HBM-traffic figure bench.py reports.

  python -m lm_head_cross_amd.prof_summary stats  KERNEL_STATS.csv  OUT.md  "<command>"
  python -m lm_head_cross_amd.prof_summary traffic FETCH.csv WRITE.csv KERNEL_SUBSTRING OUT.txt "<commands>" [KIND]
  python -m lm_head_cross_amd.prof_summary mfma   COUNTERS.csv OUT.txt "<command>"
  python -m lm_head_cross_amd.prof_summary stalls OUT.md "<commands>" PASS1.csv PASS2.csv ...

`traffic` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the same counters read for the
plain 1 GiB device copy that `bench.py --copy-calibration` runs, averages them over the dispatches of
the named kernel, and records a hash of the kernel sources, so that bench.py reports the figure only
while the kernels are unchanged.

`mfma` reads a run with the counters SQ_VALU_MFMA_BUSY_CYCLES (summed over the GPU's 1024 SIMDs)
and GRBM_GUI_ACTIVE (summed over its 8 XCDs) and reports, per kernel and grid size, the clock the
chip ran at (GRBM_GUI_ACTIVE / 8 over the dispatch's duration) and the MFMA pipe's busy fraction,
both at that clock and against 2.4 GHz (the clock behind the 2.5 PFLOP/s bf16 figure).
"""
from __future__ import annotations

import csv
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


SIMDS, XCDS, NOMINAL_HZ = 1024, 8, 2.4e9
MEASUREMENT_AIDS = ("mfma_peak.hip",)   # in csrc/ but not the head's code


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(os.listdir(csrc)):
        if name in MEASUREMENT_AIDS:
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def kernel_stats_md(stats_csv: str, title: str, command: str) -> str:
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in _rows(stats_csv):
        name = r["Name"] if len(r["Name"]) <= 70 else r["Name"][:67] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.2f}% |")
    out += ["", "Outside `orpo::`: the library GEMM (`Cijk_*`) and reduction kernels are the synthetic",
            "input generator's argmax label pass, run before any timed step; `__amd_rocclr_*` are the",
            "HIP runtime's own fills and copies (buffer setup, reading the loss back)."]
    trace = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    if os.path.exists(trace):
        groups = {}
        for r in _rows(trace):
            if "bwd_kernel" not in r["Kernel_Name"]:
                continue
            wg = int(r.get("Grid_Size_X", r.get("Grid_Size", "0"))) // int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", "512")))
            groups.setdefault(wg, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        if groups:
            out += ["", "Backward launches by grid size (workgroups): the mixed launches (coefficient tiles of",
                    "one item + dh/dW tiles of the previous) are the ones bench.py reports as `bwd`.", "",
                    "| workgroups | launches | avg (us) |", "|---|---|---|"]
            for wg in sorted(groups, reverse=True):
                v = groups[wg]
                out.append(f"| {wg} | {len(v)} | {sum(v) / len(v):.1f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(rows, counter, substr, grid=None):
    vals = [float(r["Counter_Value"]) * 1024 for r in rows
            if r["Counter_Name"] == counter and substr in r["Kernel_Name"]
            and (grid is None or int(r["Grid_Size"]) == grid)]
    return vals


def _copy_scale(rows, counter):
    vals = _per_dispatch(rows, counter, "copyBuffer")
    big = [v for v in vals if v > COPY_BYTES / 4]
    if not big:
        raise SystemExit(f"no 1 GiB copy found for {counter}: run bench.py with --copy-calibration")
    return COPY_BYTES / (sum(big) / len(big))


def traffic_txt(fetch_csv, write_csv, substr, commands, kind=None) -> str:
    fr, wr = _rows(fetch_csv), _rows(write_csv)
    fs, ws = _copy_scale(fr, "FETCH_SIZE"), _copy_scale(wr, "WRITE_SIZE")
    grid = None
    if kind is None:
        kind = substr
    else:   # the most frequent grid size of the kernel = its steady-state (mixed) launches
        sizes = [int(r["Grid_Size"]) for r in fr if substr in r["Kernel_Name"]]
        grid = max(set(sizes), key=sizes.count)
    f = _per_dispatch(fr, "FETCH_SIZE", substr, grid)
    w = _per_dispatch(wr, "WRITE_SIZE", substr, grid)
    if not f or not w:
        raise SystemExit(f"kernel {substr!r} not found")
    fetch = fs * sum(f) / len(f)
    write = ws * sum(w) / len(w)
    # Every launch kind of the head (kernel and grid size), copy-scaled, for the breakdown.
    kinds = {}
    for rows, counter, scale, col in ((fr, "FETCH_SIZE", fs, 0), (wr, "WRITE_SIZE", ws, 1)):
        for r in rows:
            if r["Counter_Name"] != counter or "orpo::" not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("orpo::", "")
            e = kinds.setdefault((name, int(r["Grid_Size"])), ([], []))
            e[col].append(float(r["Counter_Value"]) * 1024 * scale)
    table = ["", "breakdown (GB per launch, copy-scaled; kernel, grid threads, dispatches):"]
    for (name, g), (fv, wv) in sorted(kinds.items(), key=lambda kv: -sum(kv[1][0])):
        if fv and wv:
            table.append(f"  {name} | {g} | {len(fv)} | fetch {sum(fv) / len(fv) / 1e9:.3f} | "
                         f"write {sum(wv) / len(wv) / 1e9:.3f}")
    return "\n".join([
        f"kernel: {kind}",
        f"kernel_name: {substr}" + (f" (grid {grid} threads)" if grid else ""),
        f"source_hash: {source_hash()}",
        f"dispatches: {len(f)}",
        f"fetch_scale: {fs:.4f}",
        f"write_scale: {ws:.4f}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
        f"commands: {commands}",
    ] + table) + "\n"


def read_traffic(path: str):
    """(kernel, bytes per launch) if `path` exists and was taken on the current kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash():
        return None
    return kv.get("kernel"), float(kv["traffic_bytes_per_launch"])


def mfma_txt(counters_csv: str, command: str) -> str:
    per = {}   # (kernel, grid) -> dispatch id -> {counter: value, "ns": duration}
    for r in _rows(counters_csv):
        key = (r["Kernel_Name"], int(r["Grid_Size"]))
        d = per.setdefault(key, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = ["MFMA busy fraction and clock per kernel (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over 1024",
           "SIMDs; clock = GRBM_GUI_ACTIVE / 8 XCDs over the dispatch's duration).", "",
           f"command: {command}", f"source_hash: {source_hash()}", "",
           "| kernel | grid (threads) | dispatches | avg (us) | clock (GHz) | MFMA busy at that clock | "
           "MFMA busy vs 2.4 GHz |", "|---|---|---|---|---|---|---|"]
    for (name, grid), ds in sorted(per.items(), key=lambda kv: -sum(d["ns"] for d in kv[1].values())):
        ds = [d for d in ds.values() if "SQ_VALU_MFMA_BUSY_CYCLES" in d and "GRBM_GUI_ACTIVE" in d]
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds)
        if not ds or busy == 0:
            continue
        ns = sum(d["ns"] for d in ds)
        cyc = sum(d["GRBM_GUI_ACTIVE"] for d in ds) / XCDS
        short = name if len(name) <= 60 else name[:57] + "..."
        out.append(f"| `{short}` | {grid} | {len(ds)} | {ns / len(ds) / 1e3:.1f} | {cyc / ns:.3f} | "
                   f"{busy / (cyc * SIMDS):.3f} | {busy / (ns * 1e-9 * NOMINAL_HZ * SIMDS):.3f} |")
    return "\n".join(out) + "\n"


# Counters of the stall table: (counter, unit, meaning). SQ counters are summed over the GPU's
# shader engines; "quad" counters count units of 4 cycles per wave, the others cycles per CU.
STALL_COUNTERS = [
    ("SQ_VALU_MFMA_BUSY_CYCLES", "simd", "MFMA pipe busy"),
    ("SQ_VALU_MFMA_COEXEC_CYCLES", "simd", "MFMA busy while a VALU instruction issues"),
    ("SQ_ACTIVE_INST_VALU", "quad", "waves issuing VALU"),
    ("SQ_ACTIVE_INST_SCA", "quad", "waves issuing SALU / SMEM"),
    ("SQ_ACTIVE_INST_LDS", "quad", "waves issuing LDS"),
    ("SQ_ACTIVE_INST_VMEM", "quad", "waves issuing VMEM"),
    ("SQ_WAIT_INST_ANY", "quad", "waves waiting to issue (dependency, waitcnt, barrier)"),
    ("SQ_WAIT_INST_LDS", "quad", "waves waiting to issue an LDS instruction"),
    ("SQ_WAIT_ANY", "quad", "waves waiting for anything"),
    ("SQ_LDS_IDX_ACTIVE", "cu", "LDS busy with indexed (ds_*) accesses"),
    ("SQ_LDS_BANK_CONFLICT", "cu", "LDS stalled by bank conflicts"),
    ("SQ_LDS_ADDR_CONFLICT", "cu", "LDS stalled by address conflicts"),
    ("SQ_WAVE_CYCLES", "quad", "resident waves"),
]
CUS = 256


def stalls_md(csvs, command: str, kernel_substr: str = "orpo::") -> str:
    """Per kernel and grid size: each counter of STALL_COUNTERS normalised to the dispatch's own
    cycles (GRBM_GUI_ACTIVE / 8 XCDs), as a fraction of SIMD cycles (MFMA counters), of wave
    slots on a CU (quad counters x 4 / 8 waves), or of CU cycles (LDS counters)."""
    per = {}   # (kernel, grid) -> counter -> [values], plus "cyc"
    for path in csvs:
        disp = {}
        for r in _rows(path):
            if kernel_substr not in r["Kernel_Name"]:
                continue
            key = (r["Kernel_Name"], int(r["Grid_Size"]))
            disp.setdefault((key, r["Dispatch_Id"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
        for (key, _), d in disp.items():
            if "GRBM_GUI_ACTIVE" not in d:
                continue
            cyc = d["GRBM_GUI_ACTIVE"] / XCDS
            e = per.setdefault(key, {})
            for c, v in d.items():
                if c != "GRBM_GUI_ACTIVE":
                    e.setdefault(c, []).append(v / cyc)
    out = ["Where the cycles of the head's kernels go (rocprofv3 counters, one pass per 8 SQ counters;",
           "each value normalised to the dispatch's own cycles, GRBM_GUI_ACTIVE / 8 XCDs).",
           "simd = fraction of SIMD cycles (1024 SIMDs); wave = fraction of the 8 wave slots of a CU",
           "(quad-cycle counters x 4 / 8); cu = fraction of CU cycles (256 CUs).", "",
           f"commands: {command}", f"source_hash: {source_hash()}", ""]
    for (name, grid), e in sorted(per.items(), key=lambda kv: -kv[0][1]):
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in e:
            continue
        short = name if len(name) <= 70 else name[:67] + "..."
        out += [f"## `{short}` (grid {grid} threads)", "", "| counter | unit | value | meaning |",
                "|---|---|---|---|"]
        for c, unit, meaning in STALL_COUNTERS:
            if c not in e:
                continue
            v = sum(e[c]) / len(e[c])
            frac = v / (CUS * 4) if unit == "simd" else (v * 4 / (CUS * 8) if unit == "quad" else v / CUS)
            out.append(f"| {c} | {unit} | {frac:.3f} | {meaning} |")
        out.append("")
    return "\n".join(out)


def main(argv):
    if argv[1] == "stats":
        open(argv[3], "w").write(kernel_stats_md(argv[2], os.path.basename(argv[3]), argv[4]))
    elif argv[1] == "traffic":
        kind = argv[7] if len(argv) > 7 else None
        open(argv[5], "w").write(traffic_txt(argv[2], argv[3], argv[4], argv[6], kind))
    elif argv[1] == "mfma":
        open(argv[3], "w").write(mfma_txt(argv[2], argv[4]))
    elif argv[1] == "stalls":   # stalls OUT.md "<commands>" CSV...
        open(argv[2], "w").write(stalls_md(argv[4:], argv[3]))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
